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
  cpu_baseline  the oracle (test infrastructure) timed on this host on a
                bounded sample of the same workload (whole rows of C);
  per_config    the four smaller workloads, each timed the same way (context);
  attention     the attention forward on its workloads (the sequence of page
                "TileLang实战" §4.3 and a long-sequence case), timed the same
                way, with torch's scaled_dot_product_attention as context.
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
# the sources of the kernel the 8192^3 workload runs (the ring kernel and the
# helpers it includes): the committed counter record is valid while they are
# unchanged
KERNEL_SOURCES = ["tiled_gemm_03_amd/csrc/gemm_kernel.hpp", "tiled_gemm_03_amd/csrc/gemm_kernel_ring.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_f16_8192x8192x8192.json")


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def sclk_mhz():
    # rocm-smi starts through an `env python3` shebang; under a profiler's
    # preload that is an exec after GPU initialisation, so skip it there
    if "rocprof" in os.environ.get("LD_PRELOAD", "") or os.environ.get("TGEMM_NO_SCLK"):
        return None
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
        d = json.loads(r.stdout)
        for v in d.values():
            for k, s in v.items():
                if "sclk" in k.lower():
                    return s
    except Exception:
        return None
    return None


def time_calls(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    return wall * 1e3 / steps, ev


def cpu_baseline(a, b, budget_s=12.0):
    """The oracle on whole rows of C (all N columns, the full K), doubling the
    row count until the run takes budget_s seconds or more."""
    import numpy as np
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=-1, help="force a tile configuration (gemm_ex)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true")
    ap.add_argument("--no-attention", action="store_true")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only run the MFMA ceiling program (issue rate and clock of both fp16 MFMA shapes on "
                         "every SIMD, N(0,1) and all-ones operands) and print its JSON lines")
    ap.add_argument("--lds-probes", action="store_true",
                    help="only run the LDS probe program (read rate of each candidate LDS layout, direct-to-LDS "
                         "load rate of each global footprint) and print its JSON lines")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one elementwise kernel that reads and writes 512 MiB "
                         "(scale reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(a row-sharded multi-GPU product needs no collective; it is described, not built)",
              file=sys.stderr)
        sys.exit(2)

    if args.mfma_ceiling or args.lds_probes:
        # a child process of its own, started before this process touches the GPU
        from tiled_gemm_03_amd import build as B
        prog = B.CEILING_BIN if args.mfma_ceiling else B.PROBES_BIN
        if not os.path.exists(prog):
            print(f"bench.py: {prog} is not built (run __graft_entry__.build())", file=sys.stderr)
            sys.exit(1)
        sys.exit(subprocess.run([prog]).returncode)

    import numpy as np
    import torch
    import tiled_gemm_03_amd as T
    from tiled_gemm_03_amd import workloads as W

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    w = W.BY_NAME["f16_8192x8192x8192"]
    print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
    a_np, b_np = W.make_inputs(w)
    a = torch.from_numpy(a_np).to(dev)
    b = torch.from_numpy(b_np).to(dev)
    c = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)
    torch.cuda.synchronize()

    def step():
        T.gemm_tensors(a, b, c, config_id=args.config, stream=stream.cuda_stream)

    print(f"[bench] timing {args.steps} steps after {args.warmup} warmup", file=sys.stderr, flush=True)
    ms_per_step, ev = time_calls(step, args.steps, args.warmup, stream)
    flops = 2.0 * w.M * w.N * w.K
    value = flops / (ms_per_step * 1e-3) / 1e12
    kern_ms = float(np.mean(ev))
    achieved = flops / (kern_ms * 1e-3) / 1e12

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

    per_config = []
    if not args.no_per_config:
        for pw in W.WORKLOADS[:4]:
            pa, pb = W.make_inputs(pw)
            tdt = {W.F16: torch.float16, W.F32: torch.float32}
            pad = torch.from_numpy(pa).to(dev)
            pbd = torch.from_numpy(pb).to(dev)
            pc = torch.empty((pw.M, pw.N), dtype=tdt[pw.out_dtype], device=dev)
            call = lambda: T.gemm_tensors(pad, pbd, pc, stream=stream.cuda_stream)
            pms, pev = time_calls(call, 200, 20, stream)
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
            med = float(np.median(pev))
            peak = PEAK_F32_TFLOPS if pw.in_dtype == W.F32 else PEAK_F16_TFLOPS
            algo_bytes = (pw.M * pw.K + pw.K * pw.N) * (4 if pw.in_dtype == W.F32 else 2) + \
                pw.M * pw.N * (4 if pw.out_dtype == W.F32 else 2)
            pid = T.gemm_select_config(pw.M, pw.N, pw.K, pad.data_ptr(), pw.K, pbd.data_ptr(), pw.N,
                                       pc.data_ptr(), pw.N, pw.in_dtype, pw.out_dtype)
            kind = T.gemm_select_kernel(pw.M, pw.N, pw.K, pad.data_ptr(), pw.K, pbd.data_ptr(), pw.N,
                                        pc.data_ptr(), pw.N, pw.in_dtype, pw.out_dtype)
            per_config.append({
                "workload": pw.name, "config": T.gemm_config_info(pid)["name"],
                "kernel": {0: "general", 1: "tiled", 2: "ring", 3: "direct"}.get(kind, str(kind)),
                "us_median": med * 1e3, "us_p10": float(np.percentile(pev, 10)) * 1e3,
                "us_p90": float(np.percentile(pev, 90)) * 1e3, "us_per_call_wall": pms * 1e3,
                "us_back_to_back": b2b_ms * 1e3,
                "tflops": pf / (med * 1e-3) / 1e12, "frac_of_mfma_peak": pf / (med * 1e-3) / 1e12 / peak,
                "gbs": algo_bytes / (med * 1e-3) / 1e9,
                "tflops_back_to_back": pf / (b2b_ms * 1e-3) / 1e12,
                "gbs_back_to_back": algo_bytes / (b2b_ms * 1e-3) / 1e9})

    # the same 8192^3 product with column-major operands or output (gemm_t):
    # each matrix holds the same values, stored transposed
    layouts = []
    if not args.no_per_config:
        a_col = a.t().contiguous().t()
        b_col = b.t().contiguous().t()
        c_col = torch.empty((w.N, w.M), dtype=torch.float16, device=dev).t()
        kinds = {0: "general", 1: "tiled", 2: "ring", 3: "direct"}
        for name, la_, lb_, lc_ in (("A col-major", a_col, b, c), ("B col-major", a, b_col, c),
                                    ("A, B col-major", a_col, b_col, c), ("C col-major", a, b, c_col)):
            call = lambda: T.gemm_tensors(la_, lb_, lc_, stream=stream.cuda_stream)
            _, lev = time_calls(call, 20, 3, stream)
            (xa, lda_), (xb, ldb_), (xc, ldc_) = T._layout(la_), T._layout(lb_), T._layout(lc_)
            kind, lcfg = T.gemm_select_kernel_t(w.M, w.N, w.K, la_.data_ptr(), lda_, xa, lb_.data_ptr(), ldb_, xb,
                                                lc_.data_ptr(), ldc_, xc, w.in_dtype, w.out_dtype)
            med = float(np.median(lev))
            layouts.append({"layouts": name, "config": T.gemm_config_info(lcfg)["name"],
                            "kernel": kinds.get(kind, str(kind)), "us_median": med * 1e3,
                            "tflops": flops / (med * 1e-3) / 1e12})
        del a_col, b_col, c_col

    # the same product with the fused epilogue (gemm_fused)
    fused = []
    if not args.no_per_config:
        bias = torch.randn(w.N, device=dev).half()
        for name, kw in (("column bias + gelu (tanh form)", dict(bias=bias, activation=T.ACT_GELU_TANH)),
                         ("alpha 0.5, beta 1 (C read) + relu", dict(alpha=0.5, beta=1.0, activation=T.ACT_RELU))):
            call = lambda: T.gemm_tensors(a, b, c, stream=stream.cuda_stream, **kw)
            _, fev = time_calls(call, 20, 3, stream)
            med = float(np.median(fev))
            fused.append({"epilogue": name, "us_median": med * 1e3, "tflops": flops / (med * 1e-3) / 1e12})
        del bias

    # the ring kernel's edge paths on sub-views of the same operands: a K
    # tail (K not a multiple of 128) and partial column groups with C rows
    # not 4-element aligned (the fused epilogue's stores with the identity
    # epilogue); torch.matmul on the same views for context
    edges = []
    if not args.no_per_config:
        kinds = {0: "general", 1: "tiled", 2: "ring", 3: "direct"}
        for name, m_, n_, k_ in (("K tail: K = 8000", w.M, w.N, 8000),
                                 ("N = 8190, ldc = 8190 (partial groups, unaligned C rows)", w.M, 8190, w.K)):
            ea, eb = a[:m_, :k_], b[:k_, :n_]
            ec = torch.empty((m_, n_), dtype=torch.float16, device=dev)
            call = lambda: T.gemm_tensors(ea, eb, ec, stream=stream.cuda_stream)
            _, eev = time_calls(call, 20, 3, stream)
            _, tev = time_calls(lambda: torch.matmul(ea, eb, out=ec), 20, 3, stream)
            (xa, lda_), (xb, ldb_), (xc, ldc_) = T._layout(ea), T._layout(eb), T._layout(ec)
            kind, ecfg = T.gemm_select_kernel_t(m_, n_, k_, ea.data_ptr(), lda_, xa, eb.data_ptr(), ldb_, xb,
                                                ec.data_ptr(), ldc_, xc, w.in_dtype, w.out_dtype)
            med, tmed = float(np.median(eev)), float(np.median(tev))
            ef = 2.0 * m_ * n_ * k_
            edges.append({"case": name, "M": m_, "N": n_, "K": k_, "config": T.gemm_config_info(ecfg)["name"],
                          "kernel": kinds.get(kind, str(kind)), "us_median": med * 1e3,
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
            _, aev = time_calls(call, reps, max(3, reps // 10), stream)
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
                _, sev = time_calls(sdpa, reps, max(3, reps // 10), stream)
                entry["torch_sdpa_us_median"] = float(np.median(sev)) * 1e3
            except Exception as e:  # noqa: BLE001 - context only
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

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        cpu = cpu_baseline(a_np, b_np)

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
        "cpu_baseline": cpu,
        "per_config": per_config,
        "layouts_8192": layouts,
        "fused_8192": fused,
        "edges_8192": edges,
        "attention": attention,
        "sclk": sclk_mhz(),
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
