"""Benchmark of the tiled matrix product on one MI355X.

A step is one call of the library (one kernel launch) on the 8192 x 8192 x
8192 workload: fp16 inputs drawn from N(0,1) with seed 5, fp32 accumulation,
fp16 output, inputs resident in HBM before timing starts.  The metric is
TFLOP/s = 2*M*N*K / time, the formula of page "企业官网建设流程全解析" §3.4.

Printed: ONE JSON line with the contract's keys plus
  roofline      the kernel's achieved TFLOP/s from HIP events recorded around
                every launch on the stream it runs on, against MI355X's dense
                fp16 MFMA peak; `traffic` comes from the committed counter
                summary when it was taken on the current kernel source, else
                null;
  clock         shader clock, socket power, hotspot temperature and energy
                sampled by a child process (amdsmi, started before this
                process touches the GPU) during the timed steps, and the
                TFLOP/s per GHz and per watt they imply;
  cpu_baseline  the oracle (test infrastructure) timed on this host on a
                bounded sample of the same workload (whole rows of C);
  per_config    all five workloads: warm timing (back-to-back calls on the
                same inputs) and flushed timing (a 512 MiB buffer written
                between calls, so that no input or output line stays in L2 or
                the 256 MB Infinity Cache), kernel chosen, TFLOP/s, GB/s, and,
                from the CPU-baseline leg after all GPU timing, the oracle's
                GFLOP/s on the same workload and the GPU result's error
                against it (normalised as the tolerance is, plus max and mean
                absolute error);
  layouts_8192 / fused_8192 / edges_8192   the same product with column-major
                operands, the fused epilogue, and the ring kernel's edge paths;
  attention     the attention forward on its workloads, with torch's
                scaled_dot_product_attention as context.
"""
import argparse
import hashlib
import json
import math
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F16_TFLOPS = 2516.6   # 256 CU x 4096 FLOP/clk x 2.4 GHz, dense
PEAK_F32_TFLOPS = 157.3    # dense fp32 MFMA
PEAK_HBM_GBS = 8000.0
FLUSH_BYTES = 512 << 20    # written between flushed calls (2x the Infinity Cache)
# the sources of the kernel the 8192^3 workload runs (the ring kernel and the
# helpers it includes): the committed counter record is valid while they are
# unchanged
KERNEL_SOURCES = ["tiled_gemm_03_amd/csrc/gemm_kernel.hpp", "tiled_gemm_03_amd/csrc/gemm_kernel_ring.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_f16_8192x8192x8192.json")
KINDS = {0: "general", 1: "tiled", 2: "ring", 3: "direct"}


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------- clock sampler
def clock_sampler_child():
    """Child process: reads the GPU's power-management metrics table (amdsmi)
    in a loop.  Protocol on stdin: first line the PCI address of the GPU to
    sample (domain:bus:device.function, or empty when only one GPU is
    visible), then any line to stop; it then prints one JSON object with the
    samples: (monotonic seconds, current gfxclk MHz, mean of the per-XCD
    current gfxclks, average gfxclk MHz, socket power W, hotspot C, energy
    counter in microjoules, throttle status)."""
    import ctypes
    import threading
    out = {"samples": [], "error": None, "bdf": None}
    try:
        import amdsmi
        from amdsmi import amdsmi_wrapper as AW
        amdsmi.amdsmi_init(amdsmi.AmdSmiInitFlags.INIT_AMD_GPUS)
        handles = amdsmi.amdsmi_get_processor_handles()
        bdfs = [amdsmi.amdsmi_get_gpu_device_bdf(h).lower() for h in handles]
    except Exception as e:  # noqa: BLE001 - reported, not fatal
        out["error"] = f"amdsmi unavailable: {e}"
        sys.stdin.readline()
        print(json.dumps(out), flush=True)
        return
    want = sys.stdin.readline().strip().lower()
    # match domain:bus:device.function, else bus:device.function
    pick = [i for i, b in enumerate(bdfs) if want and b == want]
    pick = pick or [i for i, b in enumerate(bdfs) if want and b.split(":", 1)[-1] == want.split(":", 1)[-1]]
    if not pick and len(handles) == 1:
        pick = [0]
    if not pick:
        out["error"] = f"GPU {want!r} not among {bdfs}"
        sys.stdin.readline()
        print(json.dumps(out), flush=True)
        return
    h = handles[pick[0]]
    out["bdf"] = bdfs[pick[0]]
    stop = threading.Event()

    def waiter():
        sys.stdin.readline()
        stop.set()

    threading.Thread(target=waiter, daemon=True).start()
    gm = AW.amdsmi_gpu_metrics_t()
    acc, res, ts = ctypes.c_uint64(), ctypes.c_float(), ctypes.c_uint64()
    samples = out["samples"]
    while not stop.is_set() and len(samples) < 400000:
        t = time.monotonic()
        if AW.amdsmi_get_gpu_metrics_info(h, ctypes.byref(gm)) == 0:
            xcd = [int(c) for c in gm.current_gfxclks if 0 < c < 0xFFFF]
            e_uj = None
            if AW.amdsmi_get_energy_count(h, ctypes.byref(acc), ctypes.byref(res), ctypes.byref(ts)) == 0:
                e_uj = acc.value * float(res.value)
            samples.append((t, int(gm.current_gfxclk), sum(xcd) / len(xcd) if xcd else None,
                            int(gm.average_gfxclk_frequency), int(gm.current_socket_power),
                            int(gm.temperature_hotspot), e_uj, int(gm.throttle_status)))
        time.sleep(0.0005)
    print(json.dumps(out), flush=True)


def _valid(x, hi=0xFFFF):
    return x is not None and 0 < x < hi


def refreshes(samples):
    """The samples at which the metrics table held new values (the firmware
    refreshes it about once per second; the samples in between repeat it)."""
    out, prev = [], None
    for s in samples:
        if tuple(s[1:]) != prev:
            out.append(s)
            prev = tuple(s[1:])
    return out


def clock_window(samples, t0, t1):
    """Statistics of the table refreshes seen in [t0, t1] (monotonic
    seconds): mean / min / max of the per-XCD gfxclk (else the current
    gfxclk), socket power, hotspot temperature, and the average power from
    the energy counter between the first and last refresh of the window
    (absent where the table did not hold the value)."""
    win = [s for s in refreshes(samples) if t0 <= s[0] <= t1]
    r = {"samples": len(win), "window_ms": (t1 - t0) * 1e3}
    if not win:
        return r

    def stats(vals, key):
        vals = [v for v in vals if v is not None]
        if vals:
            r[key + "_mean"] = sum(vals) / len(vals)
            r[key + "_min"] = min(vals)
            r[key + "_max"] = max(vals)

    stats([s[2] if s[2] is not None else (s[1] if _valid(s[1]) else None) for s in win], "gfxclk_mhz")
    stats([s[3] if _valid(s[3]) else None for s in win], "avg_gfxclk_mhz")
    stats([s[4] if _valid(s[4]) else None for s in win], "socket_power_w")
    stats([s[5] if _valid(s[5]) else None for s in win], "hotspot_c")
    e = [(s[0], s[6]) for s in win if s[6] is not None]
    if len(e) >= 2 and e[-1][0] > e[0][0] and e[-1][1] >= e[0][1]:
        r["energy_power_w"] = (e[-1][1] - e[0][1]) * 1e-6 / (e[-1][0] - e[0][0])
    r["throttle_status_any"] = any(s[7] not in (0, 0xFFFFFFFF) for s in win)
    return r


class ClockSampler:
    """Parent side of clock_sampler_child.  Start it before this process
    makes any GPU call; under a profiler's preloaded library (which has
    already initialised the GPU in this process) it is not started."""

    def __init__(self, enabled=True):
        self.proc = None
        self.reason = None
        if not enabled:
            self.reason = "disabled"
        elif "rocprof" in os.environ.get("LD_PRELOAD", ""):
            self.reason = "not started under a profiler"
        else:
            try:
                self.proc = subprocess.Popen([sys.executable, os.path.abspath(__file__), "--clock-sampler"],
                                             stdin=subprocess.PIPE, stdout=subprocess.PIPE,
                                             stderr=subprocess.DEVNULL, text=True)
            except OSError as e:
                self.reason = f"could not start: {e}"
        self.data = None

    def select(self, bdf):
        if self.proc is not None:
            self.proc.stdin.write((bdf or "") + "\n")
            self.proc.stdin.flush()

    def finish(self):
        if self.proc is None:
            return {"samples": [], "error": self.reason}
        try:
            o, _ = self.proc.communicate("stop\n", timeout=60)
            self.data = json.loads(o.strip().splitlines()[-1])
        except Exception as e:  # noqa: BLE001 - reported, not fatal
            self.proc.kill()
            self.data = {"samples": [], "error": f"sampler: {e}"}
        return self.data


def device_bdf(dev_index=0):
    """PCI address of a torch device as domain:bus:device.function."""
    import torch
    p = torch.cuda.get_device_properties(dev_index)
    if all(hasattr(p, f) for f in ("pci_domain_id", "pci_bus_id", "pci_device_id")):
        return f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}.0"
    return ""


# ---------------------------------------------------------------- timing
def time_calls(fn, steps, warmup, stream, flush=None):
    """Per-call HIP-event times (ms) of `steps` calls after `warmup` calls, the
    wall time per call, and the monotonic bounds of the timed region.  With
    `flush`, it runs between calls, outside the events."""
    import torch
    for _ in range(warmup):
        if flush is not None:
            flush()
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    m0 = time.monotonic()
    t0 = time.perf_counter()
    for i in range(steps):
        if flush is not None:
            flush()
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    m1 = time.monotonic()
    ev = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return {"wall_ms_per_call": wall * 1e3 / steps, "events_ms": ev, "t0": m0, "t1": m1}


def summary_us(ev):
    import numpy as np
    return {"us_median": float(np.median(ev)) * 1e3, "us_p10": float(np.percentile(ev, 10)) * 1e3,
            "us_p90": float(np.percentile(ev, 90)) * 1e3}


def gemm_error(c, o, a, b, in_dtype):
    """The tolerance's error measure of a GPU result c against the oracle o
    (binary64, same entries): fp16 / bf16 inputs max|c - o| / (sqrt(K) max|a|
    max|b|) over the whole stored inputs (tolerance 1e-2); fp32 inputs the
    normwise max|c - o| / max|o| (tolerance 1e-4); with the absolute max and
    mean error."""
    import numpy as np
    import oracle
    from tiled_gemm_03_amd import workloads as W
    d = np.abs(c.astype(np.float64) - o)
    K = a.shape[1]
    if in_dtype == W.F32:
        e, tol = float(d.max() / max(np.abs(o).max(), 1e-300)), 1e-4
    else:
        av = np.abs(oracle.decode(a.view(np.uint16), in_dtype)).max()
        bv = np.abs(oracle.decode(b.view(np.uint16), in_dtype)).max()
        e, tol = float(d.max() / (math.sqrt(K) * av * bv)), 1e-2
    return {"normalised_max": e, "tolerance": tol, "within": bool(e <= tol and np.isfinite(c).all()),
            "max_abs": float(d.max()), "mean_abs": float(d.mean())}


def cpu_baseline(a, b, budget_s=12.0):
    """The oracle on whole rows of C (all N columns, the full K), doubling the
    row count until the run takes budget_s seconds or more."""
    import oracle
    from tiled_gemm_03_amd import workloads as W
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    M, K = a.shape
    N = b.shape[1]
    rows = 8
    while True:
        idx = W.sample_indices(M, rows, 999)
        t0 = time.perf_counter()
        oracle.gemm(a, b, W.F16, rows=idx, nthreads=threads)
        dt = time.perf_counter() - t0
        if dt >= 0.8 * budget_s or rows >= M:
            break
        rows = min(M, max(2 * rows, int(rows * budget_s / max(dt, 1e-3))))
    flops = 2.0 * rows * N * K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows} seeded rows x all {N} columns x K={K} of the 8192^3 workload "
                      f"({flops / 1e9:.1f} GFLOP, fp64 accumulation, {dt:.1f} s)",
            "seconds": dt}


def oracle_per_config(results):
    """The oracle on every workload's own inputs (full C for the four small
    ones, the 64 x 64 sampled entries of the 8192^3 one), timed on this host
    (T threads; 1 thread too on 128 x 256 x 512), and the error of the GPU
    result captured after its timing."""
    import oracle
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    for r in results:
        a, b, c_gpu = r.pop("_a"), r.pop("_b"), r.pop("_c")
        rows, cols = r.pop("_rows", None), r.pop("_cols", None)
        n_r = a.shape[0] if rows is None else len(rows)
        n_c = b.shape[1] if cols is None else len(cols)
        flops = 2.0 * n_r * n_c * a.shape[1]
        reps = max(1, int(2e8 // flops))   # repeat tiny cases to time more than a few ms
        t0 = time.perf_counter()
        for _ in range(reps):
            o = oracle.gemm(a, b, r["_in"], rows=rows, cols=cols, nthreads=threads)
        dt = (time.perf_counter() - t0) / reps
        r["oracle"] = {"gflops": flops / dt / 1e9, "threads": threads, "ms": dt * 1e3,
                       "entries": "full C" if rows is None else f"{n_r} seeded rows x {n_c} seeded columns"}
        if r["workload"] == "f16_128x256x512":
            t0 = time.perf_counter()
            for _ in range(reps):
                oracle.gemm(a, b, r["_in"], rows=rows, cols=cols, nthreads=1)
            d1 = (time.perf_counter() - t0) / reps
            r["oracle"]["gflops_1_thread"] = flops / d1 / 1e9
        r["error"] = gemm_error(c_gpu, o, a, b, r.pop("_in"))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=-1, help="force a tile configuration (gemm_ex)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true")
    ap.add_argument("--no-attention", action="store_true")
    ap.add_argument("--no-clock", action="store_true", help="do not start the clock sampler")
    ap.add_argument("--settle-ms", type=float, default=250.0,
                    help="run the product for this long before the warmup steps (and each attention workload "
                         "before its timed calls), so that the timed calls see the clock of sustained use rather "
                         "than the power controller's response to a change of load")
    ap.add_argument("--hold-ms", type=float, default=3000.0,
                    help="after the timed steps, keep running the product this long while the clock sampler reads "
                         "the metrics table (which the firmware refreshes about once per second)")
    ap.add_argument("--clock-sampler", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--dump", default=None,
                    help="write the sampler's raw samples and the per-step event times of the timed steps to "
                         "this JSON file")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one elementwise kernel that reads and writes 512 MiB "
                         "(scale reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.clock_sampler:
        clock_sampler_child()
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(a row-sharded multi-GPU product needs no collective; it is described, not built)",
              file=sys.stderr)
        sys.exit(2)

    # before anything touches the GPU
    sampler = ClockSampler(enabled=not args.no_clock)

    import numpy as np
    import torch
    import tiled_gemm_03_amd as T
    from tiled_gemm_03_amd import workloads as W

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sampler.select(device_bdf(0))
    w = W.BY_NAME["f16_8192x8192x8192"]
    print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
    a_np, b_np = W.make_inputs(w)
    a = torch.from_numpy(a_np).to(dev)
    b = torch.from_numpy(b_np).to(dev)
    c = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)
    torch.cuda.synchronize()

    def step():
        T.gemm_tensors(a, b, c, config_id=args.config, stream=stream.cuda_stream)

    # settle: leave the idle clock state before the warmup steps (the power
    # controller's response to a burst from idle makes steps 2-50 up to 40%
    # slower than sustained use)
    settle_steps = 0
    load0 = time.monotonic()   # the product runs without pause from here to the end of the hold
    ts0 = time.perf_counter()
    while (time.perf_counter() - ts0) * 1e3 < args.settle_ms:
        for _ in range(10):
            step()
        settle_steps += 10
        torch.cuda.synchronize()
    settle = {"ms": (time.perf_counter() - ts0) * 1e3, "steps": settle_steps}
    print(f"[bench] settled for {settle['ms']:.0f} ms ({settle_steps} steps); timing {args.steps} steps after "
          f"{args.warmup} warmup", file=sys.stderr, flush=True)
    mw0 = time.monotonic()
    main_t = time_calls(step, args.steps, args.warmup, stream)
    # hold: the same product, untimed, while the sampler reads the table
    th0 = time.monotonic()
    hold_steps = 0
    while (time.monotonic() - th0) * 1e3 < args.hold_ms:
        for _ in range(10):
            step()
        hold_steps += 10
        torch.cuda.synchronize()
    th1 = time.monotonic()
    ms_per_step = main_t["wall_ms_per_call"]
    ev = main_t["events_ms"]
    flops = 2.0 * w.M * w.N * w.K
    value = flops / (ms_per_step * 1e-3) / 1e12
    kern_ms = float(np.mean(ev))
    achieved = flops / (kern_ms * 1e-3) / 1e12
    print(f"[bench] {value:.1f} TFLOP/s ({ms_per_step:.4f} ms per step), kernel {achieved:.1f} TFLOP/s",
          file=sys.stderr, flush=True)
    # the sampled entries of the timed product's output, for the error check
    rows5, cols5 = W.sample_indices(w.M, 64, w.seed + 100), W.sample_indices(w.N, 64, w.seed + 200)
    c5 = c[torch.from_numpy(rows5).to(dev)][:, torch.from_numpy(cols5).to(dev)].cpu().numpy()

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        try:
            with open(TRAFFIC_FILE) as f:
                tr = json.load(f)
            if tr.get("kernel_source_hash") == kernel_source_hash():
                traffic = tr.get("hbm_bytes_per_launch")
        except Exception:
            traffic = None

    cfg_id = T.gemm_select_config(w.M, w.N, w.K, a.data_ptr(), w.K, b.data_ptr(), w.N, c.data_ptr(), w.N,
                                  w.in_dtype, w.out_dtype) if args.config < 0 else args.config
    info = T.gemm_config_info(cfg_id)

    flush_buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
    flush_val = [0]

    def flush():
        flush_val[0] += 1
        flush_buf.fill_(flush_val[0])

    per_config = []
    if not args.no_per_config:
        tdt = {W.F16: torch.float16, W.F32: torch.float32}
        for pw in W.WORKLOADS[:4]:
            pa, pb = W.make_inputs(pw)
            pad = torch.from_numpy(pa).to(dev)
            pbd = torch.from_numpy(pb).to(dev)
            pc = torch.empty((pw.M, pw.N), dtype=tdt[pw.out_dtype], device=dev)
            call = lambda: T.gemm_tensors(pad, pbd, pc, stream=stream.cuda_stream)
            warm = time_calls(call, 200, 20, stream)
            cold = time_calls(call, 100, 5, stream, flush=flush)
            # back to back: events around 200 launches in a row (the launch
            # latency of one call overlaps the previous kernel)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(200):
                call()
            e1.record(stream)
            torch.cuda.synchronize()
            b2b_ms = e0.elapsed_time(e1) / 200
            pf = 2.0 * pw.M * pw.N * pw.K
            peak = PEAK_F32_TFLOPS if pw.in_dtype == W.F32 else PEAK_F16_TFLOPS
            algo_bytes = (pw.M * pw.K + pw.K * pw.N) * (4 if pw.in_dtype == W.F32 else 2) + \
                pw.M * pw.N * (4 if pw.out_dtype == W.F32 else 2)
            pid = T.gemm_select_config(pw.M, pw.N, pw.K, pad.data_ptr(), pw.K, pbd.data_ptr(), pw.N,
                                       pc.data_ptr(), pw.N, pw.in_dtype, pw.out_dtype)
            kind = T.gemm_select_kernel(pw.M, pw.N, pw.K, pad.data_ptr(), pw.K, pbd.data_ptr(), pw.N,
                                        pc.data_ptr(), pw.N, pw.in_dtype, pw.out_dtype)
            entry = {"workload": pw.name, "config": T.gemm_config_info(pid)["name"], "kernel": KINDS.get(kind, kind),
                     "algorithmic_flop": pf, "algorithmic_bytes": algo_bytes,
                     "us_per_call_wall": warm["wall_ms_per_call"] * 1e3, "us_back_to_back": b2b_ms * 1e3}
            for mode, t in (("warm", warm), ("flushed", cold)):
                s = summary_us(t["events_ms"])
                sec = s["us_median"] * 1e-6
                s.update({"tflops": pf / sec / 1e12, "frac_of_mfma_peak": pf / sec / 1e12 / peak,
                          "gbs": algo_bytes / sec / 1e9, "frac_of_hbm_peak": algo_bytes / sec / 1e9 / PEAK_HBM_GBS})
                entry[mode] = s
            entry["tflops_back_to_back"] = pf / (b2b_ms * 1e-3) / 1e12
            entry.update({"_a": pa, "_b": pb, "_c": pc.cpu().numpy(), "_in": pw.in_dtype})
            per_config.append(entry)
            del pad, pbd, pc
        # the 8192^3 workload itself: its warm figures are the main timing's;
        # flushed: 20 calls with the flush between them
        cold = time_calls(step, 20, 3, stream, flush=flush)
        s_w = summary_us(ev)
        s_c = summary_us(cold["events_ms"])
        entry = {"workload": w.name, "config": info["name"], "kernel": "ring", "algorithmic_flop": flops,
                 "algorithmic_bytes": (w.M * w.K + w.K * w.N + w.M * w.N) * 2}
        for mode, s in (("warm", s_w), ("flushed", s_c)):
            sec = s["us_median"] * 1e-6
            s.update({"tflops": flops / sec / 1e12, "frac_of_mfma_peak": flops / sec / 1e12 / PEAK_F16_TFLOPS})
            entry[mode] = s
        entry.update({"_a": a_np, "_b": b_np, "_c": c5, "_rows": rows5, "_cols": cols5, "_in": w.in_dtype})
        per_config.append(entry)
    else:
        per_config.append({"workload": w.name, "_a": a_np, "_b": b_np, "_c": c5, "_rows": rows5, "_cols": cols5,
                           "_in": w.in_dtype})
    del flush_buf

    # the same 8192^3 product with column-major operands or output (gemm_t):
    # each matrix holds the same values, stored transposed
    layouts = []
    if not args.no_per_config:
        a_col = a.t().contiguous().t()
        b_col = b.t().contiguous().t()
        c_col = torch.empty((w.N, w.M), dtype=torch.float16, device=dev).t()
        for name, la_, lb_, lc_ in (("A col-major", a_col, b, c), ("B col-major", a, b_col, c),
                                    ("A, B col-major", a_col, b_col, c), ("C col-major", a, b, c_col)):
            call = lambda: T.gemm_tensors(la_, lb_, lc_, stream=stream.cuda_stream)
            lev = time_calls(call, 20, 3, stream)["events_ms"]
            (xa, lda_), (xb, ldb_), (xc, ldc_) = T._layout(la_), T._layout(lb_), T._layout(lc_)
            kind, lcfg = T.gemm_select_kernel_t(w.M, w.N, w.K, la_.data_ptr(), lda_, xa, lb_.data_ptr(), ldb_, xb,
                                                lc_.data_ptr(), ldc_, xc, w.in_dtype, w.out_dtype)
            med = float(np.median(lev))
            layouts.append({"layouts": name, "config": T.gemm_config_info(lcfg)["name"],
                            "kernel": KINDS.get(kind, kind), "us_median": med * 1e3,
                            "tflops": flops / (med * 1e-3) / 1e12})
        del a_col, b_col, c_col

    # the same product with the fused epilogue (gemm_fused)
    fused = []
    if not args.no_per_config:
        bias = torch.randn(w.N, device=dev).half()
        for name, kw in (("column bias + gelu (tanh form)", dict(bias=bias, activation=T.ACT_GELU_TANH)),
                         ("alpha 0.5, beta 1 (C read) + relu", dict(alpha=0.5, beta=1.0, activation=T.ACT_RELU))):
            call = lambda: T.gemm_tensors(a, b, c, stream=stream.cuda_stream, **kw)
            fev = time_calls(call, 20, 3, stream)["events_ms"]
            med = float(np.median(fev))
            fused.append({"epilogue": name, "us_median": med * 1e3, "tflops": flops / (med * 1e-3) / 1e12})
        # an 8-bit output (OCP E4M3) with the same epilogue
        c8 = torch.empty((w.M, w.N), dtype=torch.float8_e4m3fn, device=dev)
        call = lambda: T.gemm_tensors(a, b, c8, stream=stream.cuda_stream, alpha=1.0 / 64, bias=bias,
                                      activation=T.ACT_GELU_TANH)
        fev = time_calls(call, 20, 3, stream)["events_ms"]
        med = float(np.median(fev))
        fused.append({"epilogue": "alpha 1/64, column bias + gelu (tanh form), fp8 e4m3 output",
                      "us_median": med * 1e3, "tflops": flops / (med * 1e-3) / 1e12})
        del c8
        # the identity epilogue (what an unaligned C or N % 4 != 0 runs)
        call = lambda: T.gemm_tensors(a, b, c, stream=stream.cuda_stream, alpha=1.0)
        fev = time_calls(call, 20, 3, stream)["events_ms"]
        med = float(np.median(fev))
        fused.append({"epilogue": "identity (alpha 1)", "us_median": med * 1e3, "tflops": flops / (med * 1e-3) / 1e12})
        # the plain product again, right after, for the comparison at the same clock
        pev = time_calls(step, 20, 3, stream)["events_ms"]
        med = float(np.median(pev))
        fused.append({"epilogue": "none (plain, same run)", "us_median": med * 1e3,
                      "tflops": flops / (med * 1e-3) / 1e12})
        del bias

    # the ring kernel's edge paths on sub-views of the same operands: a K
    # tail (K not a multiple of 128) and partial column groups with C rows
    # not 4-element aligned (the fused epilogue's stores with the identity
    # epilogue); torch.matmul on the same views for context
    edges = []
    if not args.no_per_config:
        for name, m_, n_, k_ in (("K tail: K = 8000", w.M, w.N, 8000),
                                 ("N = 8190, ldc = 8190 (partial groups, unaligned C rows)", w.M, 8190, w.K)):
            ea, eb = a[:m_, :k_], b[:k_, :n_]
            ec = torch.empty((m_, n_), dtype=torch.float16, device=dev)
            call = lambda: T.gemm_tensors(ea, eb, ec, stream=stream.cuda_stream)
            eev = time_calls(call, 20, 3, stream)["events_ms"]
            tev = time_calls(lambda: torch.matmul(ea, eb, out=ec), 20, 3, stream)["events_ms"]
            (xa, lda_), (xb, ldb_), (xc, ldc_) = T._layout(ea), T._layout(eb), T._layout(ec)
            kind, ecfg = T.gemm_select_kernel_t(m_, n_, k_, ea.data_ptr(), lda_, xa, eb.data_ptr(), ldb_, xb,
                                                ec.data_ptr(), ldc_, xc, w.in_dtype, w.out_dtype)
            med, tmed = float(np.median(eev)), float(np.median(tev))
            ef = 2.0 * m_ * n_ * k_
            edges.append({"case": name, "M": m_, "N": n_, "K": k_, "config": T.gemm_config_info(ecfg)["name"],
                          "kernel": KINDS.get(kind, kind), "us_median": med * 1e3,
                          "tflops": ef / (med * 1e-3) / 1e12, "torch_matmul_us_median": tmed * 1e3})
            del ec

    # the attention forward (attention_fwd) on its workloads: O = softmax(scale
    # Q K^T) V per head, fp16, inputs resident; FLOPs of the two products over
    # the visible (query, key) pairs, HBM bytes of Q, K, V and O once
    attention = []
    if not args.no_attention:
        for aw in W.ATTN_WORKLOADS:
            g = torch.Generator(device="cpu").manual_seed(11)
            shape = (aw.B, aw.H, aw.N, aw.d)
            q_ = torch.randn(shape, generator=g).half().to(dev)
            k_ = torch.randn(shape, generator=g).half().to(dev)
            v_ = torch.randn(shape, generator=g).half().to(dev)
            o_ = torch.empty_like(q_)
            call = lambda: T.attention_tensors(q_, k_, v_, o_, scale=aw.scale, causal=aw.causal,
                                               stream=stream.cuda_stream)
            reps = 200 if aw.N <= 1024 else 20
            # settle on this kernel's own sustained clock (the product before
            # it leaves the power controller at the product's clock), as the
            # product itself settles before its steps
            ts0 = time.perf_counter()
            while (time.perf_counter() - ts0) * 1e3 < args.settle_ms:
                for _ in range(5):
                    call()
                torch.cuda.synchronize()
            aev = time_calls(call, reps, max(3, reps // 10), stream)["events_ms"]
            med = float(np.median(aev))
            af = aw.flops()
            abytes = 4 * aw.B * aw.H * aw.N * aw.d * 2
            entry = {"workload": aw.name, "B": aw.B, "H": aw.H, "N": aw.N, "d": aw.d, "causal": aw.causal,
                     "scale": aw.scale, "tile_rows_over_32": T.attention_waves(aw.B, aw.H, aw.N, aw.d),
                     "us_median": med * 1e3, "tflops": af / (med * 1e-3) / 1e12,
                     "frac_of_mfma_peak": af / (med * 1e-3) / 1e12 / PEAK_F16_TFLOPS,
                     "gbs": abytes / (med * 1e-3) / 1e9, "algorithmic_flop": af, "algorithmic_bytes": abytes}
            # context: torch's own scaled_dot_product_attention on the same tensors
            sdpa = lambda: torch.nn.functional.scaled_dot_product_attention(q_, k_, v_, is_causal=aw.causal,
                                                                            scale=aw.scale)
            try:
                sev = time_calls(sdpa, reps, max(3, reps // 10), stream)["events_ms"]
                entry["torch_sdpa_us_median"] = float(np.median(sev)) * 1e3
            except Exception:  # noqa: BLE001 - context only
                entry["torch_sdpa_us_median"] = None
            attention.append(entry)
            del q_, k_, v_, o_

    if args.calibrate_copy:
        src = torch.ones(128 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print("[bench] calibration: neg over 512 MiB in, 512 MiB out", file=sys.stderr, flush=True)
        del src, dst

    # every GPU measurement is done: the clock record, then the CPU leg
    sd = sampler.finish()
    clock = {"source": "amdsmi GPU metrics table, read by a child process every ~0.5 ms",
             "bdf": sd.get("bdf"), "error": sd.get("error")}
    if sd.get("samples"):
        clock["table_refresh_ms_median"] = None
        rf = [x[0] for x in refreshes(sd["samples"])]
        if len(rf) >= 3:
            clock["table_refresh_ms_median"] = float(np.median(np.diff(rf))) * 1e3
        clock["timed_steps"] = clock_window(sd["samples"], main_t["t0"], main_t["t1"])
        # the product kept running right after the timed steps: the refreshes
        # of that window give the clock and power of sustained use (the
        # table lags: a refresh within about a period of the start of the
        # load can still hold idle values, so those are left out)
        tw = clock_window(sd["samples"], max(th0, load0 + 1.2), th1)
        tw["steps"] = hold_steps
        clock["hold_after_timed"] = tw
        g = tw.get("gfxclk_mhz_mean")
        if g:
            # the dense fp16 rate at the clock the timed steps ran at
            dense = 256 * 4096 * g * 1e6 / 1e12
            clock["dense_fp16_tflops_at_clock"] = dense
            clock["kernel_frac_of_dense_at_clock"] = achieved / dense
            clock["note"] = ("the table refreshes about once per second, so the timed steps (tens of ms) see at "
                             "most one refresh; the clock of the hold window (the same product, right after) stands "
                             "for theirs")
        pw_ = tw.get("energy_power_w") or tw.get("socket_power_w_mean")
        if pw_:
            clock["kernel_tflops_per_watt"] = achieved / pw_

    if args.dump:
        with open(args.dump, "w") as f:
            json.dump({"samples": sd.get("samples"), "t_warmup": mw0, "t0": main_t["t0"], "t1": main_t["t1"],
                       "events_ms": ev}, f)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] oracle on every workload (errors, GFLOP/s)", file=sys.stderr, flush=True)
        oracle_per_config(per_config)
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        cpu = cpu_baseline(a_np, b_np)
    for r in per_config:
        for k in [k for k in r if k.startswith("_")]:
            del r[k]
    if args.no_per_config:
        per_config = [r for r in per_config if len(r) > 1]
    err5 = next((r.get("error") for r in per_config if r.get("workload") == w.name), None)

    line = {
        "metric": "GEMM TFLOP/s (fp16 in, fp32 acc) at 8192^3 and % of MI355X MFMA peak",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": "f16_8192x8192x8192: C = A x B, row-major, A,B ~ N(0,1) seed 5 cast to fp16, "
                               "fp32 accumulation, fp16 output",
                   "M": w.M, "N": w.N, "K": w.K, "accumulate": "f32", "out_dtype": "f16",
                   "tile_config": info["name"], "parallelism": "single GPU"},
        "frac_of_mfma_peak": value / PEAK_F16_TFLOPS,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_F16_TFLOPS, "traffic": traffic,
                     "kernel_ms_mean": kern_ms, "kernel_ms_p10": float(np.percentile(ev, 10)),
                     "kernel_ms_p90": float(np.percentile(ev, 90)),
                     "algorithmic_flop_per_launch": flops,
                     "algorithmic_bytes_per_launch": (w.M * w.K + w.K * w.N + w.M * w.N) * 2},
        "settle": settle,
        "events_ms_first_last": [ev[0], ev[-1]],
        "clock": clock,
        "error_8192_sampled": err5,
        "cpu_baseline": cpu,
        "per_config": per_config,
        "layouts_8192": layouts,
        "fused_8192": fused,
        "edges_8192": edges,
        "attention": attention,
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
