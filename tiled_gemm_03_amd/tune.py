"""Offline configuration search that writes the library's exact-call table.

The method is the one the DeepSeek/Ascend TileLang toolkit page describes in
its closing advice (§6) and its tuning table (§4.3): screen the configuration
space quickly on a small problem (M = N = K = 1024), keep the five best
candidates, then time those at the real sizes and keep the fastest; tune
with a realistic data distribution (N(0,1) here: all-zero data runs at a
higher clock and gives numbers that do not hold).  The candidates are the
library's tile configurations (`gemm_ex`'s config_id: each is a tile-config
tuple block_M, block_N, block_K, num_stages, waves of page
"企业官网建设流程全解析", §3.3), restricted to the input type's family.

Output: `csrc/tuned_table.inc`, one line per tuned call
    {M, N, K, lda, ldb, ldc, in_dtype, out_dtype, config},
which `table_choice` in tgemm.hip consults before its rule (exact matches of
row-major calls only; rebuild the library afterwards), and a JSON record of
every timing.

Usage (on an MI355X, with the library built):
    python -m tiled_gemm_03_amd.tune [--shapes M,N,K,in,out[,lda,ldb,ldc] ...]
                                     [--emit] [--json FILE]
Without --shapes it tunes the five workloads of the benchmark table.
"""
import argparse
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
TABLE = os.path.join(HERE, "csrc", "tuned_table.inc")
SCREEN = (1024, 1024, 1024)
KEEP = 5


def _time(call, stream, reps):
    """Median kernel time (ms) of `reps` launches, HIP events on `stream`."""
    import torch
    call()
    torch.cuda.synchronize()
    ev = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev]))


def _operands(M, N, K, in_dt, out_dt, lda, ldb, ldc, seed=0):
    """N(0,1) operands rounded to the input type, in storage with the given
    leading dimensions (views of wider tensors)."""
    import torch
    from . import workloads as W
    tdt = {W.F32: torch.float32, W.F16: torch.float16, W.BF16: torch.bfloat16}
    g = torch.Generator(device="cpu").manual_seed(seed)
    a = torch.randn(M, lda, generator=g).to(tdt[in_dt]).cuda()[:, :K]
    b = torch.randn(K, ldb, generator=g).to(tdt[in_dt]).cuda()[:, :N]
    c = torch.empty(M, ldc, dtype=tdt[out_dt], device="cuda")[:, :N]
    return a, b, c


def candidates(in_dt):
    from . import F32, gemm_config_info, gemm_num_configs
    fam = F32 if in_dt == F32 else 1
    return [i for i in range(gemm_num_configs()) if gemm_config_info(i)["in_dtype"] == fam]


def time_configs(spec, configs, reps):
    """{config: ms} for one call spec (M, N, K, in, out, lda, ldb, ldc)."""
    import torch
    from . import gemm_tensors
    M, N, K, in_dt, out_dt, lda, ldb, ldc = spec
    a, b, c = _operands(M, N, K, in_dt, out_dt, lda, ldb, ldc)
    stream = torch.cuda.current_stream()
    out = {}
    for cid in configs:
        out[cid] = _time(lambda: gemm_tensors(a, b, c, config_id=cid, stream=stream.cuda_stream), stream, reps)
    return out


def current_choice(spec):
    """The configuration the built library's table picks for a call spec
    (host-only lookup, with distinct aligned stand-in addresses)."""
    from . import gemm_select_config
    M, N, K, in_dt, out_dt, lda, ldb, ldc = spec
    base = 1 << 40
    return gemm_select_config(M, N, K, base, lda, base + (1 << 36), ldb, base + (2 << 36), ldc, in_dt, out_dt)


def tune(specs, reps=20, log=print):
    """Screen at 1024^3 per type pair, refine the best KEEP at each spec."""
    record = {"screen": {}, "refine": []}
    entries = []
    screened = {}
    for spec in specs:
        in_dt, out_dt = spec[3], spec[4]
        if (in_dt, out_dt) not in screened:
            s = (*SCREEN, in_dt, out_dt, SCREEN[2], SCREEN[1], SCREEN[1])
            t = time_configs(s, candidates(in_dt), reps)
            ranked = sorted(t, key=t.get)[:KEEP]
            screened[(in_dt, out_dt)] = ranked
            record["screen"][f"{in_dt}-{out_dt}"] = {str(k): v * 1e3 for k, v in t.items()}  # us
            log(f"[tune] screen {in_dt}->{out_dt} at {SCREEN}: " +
                ", ".join(f"cfg{k} {t[k] * 1e3:.1f} us" for k in sorted(t, key=t.get)))
        # the configuration the library picks now is always refined too: a
        # tile that is slow at the screening size (the 256 x 256 tile has 16
        # tiles at 1024^3) may still be the best at the real size
        cands = list(screened[(in_dt, out_dt)])
        cur = current_choice(spec)
        if cur >= 0 and cur not in cands:
            cands.append(cur)
        t = time_configs(spec, cands, reps)
        best = min(t, key=t.get)
        record["refine"].append({"spec": list(spec), "us": {str(k): v * 1e3 for k, v in t.items()}, "best": best})
        entries.append((*spec, best))
        log(f"[tune] {spec}: best cfg{best} ({t[best] * 1e3:.1f} us); " +
            ", ".join(f"cfg{k} {v * 1e3:.1f}" for k, v in sorted(t.items(), key=lambda kv: kv[1])))
    return entries, record


def emit(entries, path=TABLE, note=""):
    """Writes the exact-call table included by tgemm.hip."""
    lines = ["// tuned_table.inc -- exact-call entries written by tiled_gemm_03_amd/tune.py (the",
             "// configuration search: screen at M = N = K = 1024, refine the best five and the current choice",
             "// at the real size).",
             f"// {note}".rstrip(),
             "// {M, N, K, lda, ldb, ldc, in_dtype, out_dtype, config}"]
    for M, N, K, in_dt, out_dt, lda, ldb, ldc, cfg in entries:
        lines.append(f"{{{M}, {N}, {K}, {lda}, {ldb}, {ldc}, {in_dt}, {out_dt}, {cfg}}},")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def default_specs():
    from . import workloads as W
    out = []
    for w in W.WORKLOADS:
        # the benchmark's operands: tight leading dimensions
        out.append((w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.K, w.N, w.N))
    return out


def parse_spec(s):
    v = [int(x) for x in s.split(",")]
    if len(v) == 5:
        M, N, K, i, o = v
        return (M, N, K, i, o, K, N, N)
    if len(v) == 8:
        return tuple(v)
    raise ValueError(f"bad shape spec {s!r}: M,N,K,in,out[,lda,ldb,ldc]")


def main(argv=None):
    # torch first: it brings its HIP runtime, which the library then shares
    import torch  # noqa: F401
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--shapes", nargs="*", type=parse_spec)
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--emit", action="store_true", help=f"write the table ({TABLE} unless --table)")
    ap.add_argument("--table", default=TABLE, help="where --emit writes the table")
    ap.add_argument("--json", help="write every timing to this file")
    args = ap.parse_args(argv)
    specs = args.shapes or default_specs()
    entries, record = tune(specs, args.reps, log=lambda m: print(m, flush=True))
    if args.emit:
        import torch
        emit(entries, path=args.table, note=f"measured on {torch.cuda.get_device_name(0)}")
        print(f"[tune] wrote {args.table}; rebuild the library to use it", flush=True)
    if args.json:
        with open(args.json, "w") as f:
            json.dump(record, f, indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
