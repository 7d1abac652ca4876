#!/usr/bin/env python3
"""Benchmark of the NF4 + LoRA linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config layer_70b]

A step is one training pass over one batch: forward (U = X A^T,
Y = X W'^T + s U B^T) and backward (dU, dB, dA, dX) through the C ABI for
every linear of the workload, with every input already in HBM.  Quantization
happens once before timing (the method quantizes at load time) and is reported
separately as quantize_ms.  The default workload is the largest one that fits
one GPU: one 70B-class decoder layer, seven NF4 linears (q, o 8192x8192; k, v
1024x8192; gate, up 28672x8192; down 8192x28672), T = 4096 tokens, r = 64,
alpha = 16.  ``--config small_token`` times the forward alone, as that
workload is defined.

Prints one JSON line: throughput in TFLOP/s of algorithmic work
(fwd 2TNK + 2Tr(K+N), bwd 2TNK + 4Tr(K+N)), the 4-bit weight-stream GB/s, a
roofline entry for the dominant kernel timed live by events its own dispatch
stamps (average, median, p10 and p90 per launch), a dense bf16 GEMM of the same
shapes as context, and the CPU oracle timed on a bounded sample.  The K timed
steps run without those events (a launch that carries them costs the host about
25 us more); the per-kernel times come from K more steps of the same workload
run right after them with the events on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NF4+LoRA linear fwd+bwd TFLOP/s and 4-bit weight GB/s, % of MI355X roofline"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E
WORKLOAD_TEXT = {
    "attn_4096": "attention projection: NF4 W 4096x4096 (block 64, double-quant groups of 256), T=2048, r=16, alpha=32",
    "mlp_8b": "8B-class MLP: gate/up 14336x4096, down 4096x14336, NF4 with 1% outliers, T=4096, r=64, alpha=16",
    "layer_70b": "70B-class layer: q,o 8192x8192, k,v 1024x8192, gate/up 28672x8192, down 8192x28672, T=4096, r=64",
    "small_token": "small-token forward: NF4 W {n}x8192, T={t}, r=16, alpha=32",
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0,
                    help="timed steps (default: 100, or 500 for the microsecond-scale small_token forward)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="layer_70b", choices=["attn_4096", "mlp_8b", "layer_70b", "small_token"])
    ap.add_argument("--tokens", type=int, default=1, help="T for --config small_token")
    ap.add_argument("--wide", action="store_true", help="28672x8192 instead of 8192x8192 for small_token")
    ap.add_argument("--copies", type=int, default=0,
                    help="rotating input/weight copies; default: enough for 512 MB, twice the 256 MB MALL")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="LoRA dropout probability on the adapter input (training configs; default 0: none)")
    ap.add_argument("--adamw", action="store_true",
                    help="end each training step with the fused AdamW update of every A and B (timed as 'adamw')")
    ap.add_argument("--adamw8", action="store_true",
                    help="the same with block-wise 8-bit moments (timed as 'adamw8')")
    ap.add_argument("--adapters", type=int, default=0,
                    help="serve the forward with this many adapters of a pool, the tokens cut into as many equal "
                         "segments (many-adapter batching; forward only)")
    ap.add_argument("--merge", action="store_true",
                    help="time the export merge W' + s B A (NF4 base, bf16 out) of every linear instead of a step")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-context-gemm", action="store_true",
                    help="skip the dense bf16 torch.mm of the same shapes (context for the fused GEMMs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 256 MiB (scales rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    ap.add_argument("--traffic-from", metavar="DIR",
                    help="write profiles/traffic_<kernel>_<workload>.json from rocprofv3 --pmc outputs under DIR "
                         "(subdirectories fetch/, write/ of this bench command and calib_fetch/, calib_write/ of "
                         "--calibrate-copy) and exit")
    ap.add_argument("--traffic-kernel", default=None, help="kernel for --traffic-from (default: the timed GEMMs)")
    ap.add_argument("--traffic-command", default="", help="the profiled command, recorded in the JSON")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


KERNEL_SOURCES = {"nf4_gemm_fwd": "nf4_gemm.hip", "nf4_gemm_dx": "nf4_gemm.hip", "nf4_gemv": "nf4_gemv.hip",
                  "merge": "merge.hip"}
# kernel symbols behind each timed launch label (the small-token forward has two kernels)
KERNEL_SYMBOLS = {"nf4_gemm_fwd": ("k_nf4_gemm_fwd",), "nf4_gemm_dx": ("k_nf4_gemm_dx",),
                  "nf4_gemv": ("k_nf4_gemv", "k_nf4_gemv_rows", "k_nf4_gemv_mrows", "k_nf4_gemv_m32")}


def _code_only(text: str) -> str:
    """Source text without comments and with whitespace runs collapsed (what the compiler sees)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return re.sub(r"\s+", " ", text).strip()


def source_digest(kernel: str) -> str:
    """Digest of the code a kernel is built from (a counter summary is valid only for it; comments and
    layout do not count)."""
    h = hashlib.sha256()
    for name in (KERNEL_SOURCES[kernel], "device.h"):
        with open(os.path.join(ROOT, "bit_quantized_lora_02_amd", "csrc", name), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_path(kernel: str, workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")


def traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes per launch from a committed counter summary, if it matches the current kernel source."""
    path = traffic_path(kernel, workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_digest") != source_digest(kernel):
        return None
    return d.get("hbm_bytes_per_launch")


def _pmc_rows(directory: str):
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"no rocprofv3 counter_collection.csv under {directory}")
    return rows


def _per_dispatch_kib(rows, counter: str, match) -> list:
    """Counter value (KiB) of every dispatch whose kernel name satisfies `match`."""
    per = {}
    for r in rows:
        if r["Counter_Name"] != counter or not match(r["Kernel_Name"]):
            continue
        key = (r.get("Dispatch_Id") or r.get("Correlation_Id") or len(per))
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    return list(per.values())


def write_traffic(args, workload: str, kernels):
    """HBM traffic per launch from FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by what the
    same counter reads for a plain device copy of known size."""
    d = args.traffic_from
    calib_bytes = 256 << 20
    cf = _per_dispatch_kib(_pmc_rows(os.path.join(d, "calib_fetch")), "FETCH_SIZE", lambda n: "opy" in n)
    cw = _per_dispatch_kib(_pmc_rows(os.path.join(d, "calib_write")), "WRITE_SIZE", lambda n: "opy" in n)
    cf = [v for v in cf if v > calib_bytes / 1024 / 8]
    cw = [v for v in cw if v > calib_bytes / 1024 / 8]
    if not cf or not cw:
        raise SystemExit("calibration copy dispatches not found")
    f_fac = calib_bytes / (sum(cf) / len(cf) * 1024)
    w_fac = calib_bytes / (sum(cw) / len(cw) * 1024)
    fetch_rows = _pmc_rows(os.path.join(d, "fetch"))
    write_rows = _pmc_rows(os.path.join(d, "write"))
    for k in kernels:
        syms = KERNEL_SYMBOLS.get(k, ("k_" + k,))
        match = lambda n: any(sy + "<" in n or sy + "(" in n for sy in syms)
        fk = _per_dispatch_kib(fetch_rows, "FETCH_SIZE", match)
        wk = _per_dispatch_kib(write_rows, "WRITE_SIZE", match)
        if not fk or not wk:
            log(f"no dispatches of {' or '.join(syms)} in the counter runs")
            continue
        fetch_b = sum(fk) / len(fk) * 1024 * f_fac
        write_b = sum(wk) / len(wk) * 1024 * w_fac
        out = {"kernel": k, "workload": workload, "source_digest": source_digest(k),
               "hbm_bytes_per_launch": fetch_b + write_b, "fetch_bytes_per_launch": fetch_b,
               "write_bytes_per_launch": write_b, "fetch_kib_per_dispatch": sum(fk) / len(fk),
               "write_kib_per_dispatch": sum(wk) / len(wk), "dispatches": [len(fk), len(wk)],
               "fetch_scale": f_fac, "write_scale": w_fac,
               "calibration": "torch device copy of 256 MiB (python bench.py --calibrate-copy)",
               "command": args.traffic_command}
        with open(traffic_path(k, workload), "w") as f:
            json.dump(out, f, indent=1)
            f.write("\n")
        print(json.dumps(out))


def linears_for(args):
    from bit_quantized_lora_02_amd.synth import CONFIGS
    c = CONFIGS[args.config]
    if args.config == "small_token":
        name, n_out, n_in = c["linears"][1 if args.wide else 0]
        return [(name, n_out, n_in)], args.tokens, c["r"], c["alpha"], c["outliers"], False
    return c["linears"], c["T"], c["r"], c["alpha"], c["outliers"], True


def cpu_baseline(inps, train: bool, target_s: float, slice_cap: int):
    """The oracle as it is (binary64 C, OpenMP over the host cores) on a bounded sample of the workload.

    Every linear's weight is quantized in full, as at load time.  Then every linear runs forward (and,
    for training workloads, backward) on the first ts tokens, ts <= slice_cap, sized so that the whole
    leg takes about target_s; each pass also dequantizes its weight once.  The contractions are linear in
    T and the dequantization is not, so the full step's CPU time is extrapolated as
    passes x dequantize + slice time x T / ts, and marked as extrapolated when ts < T."""
    import oracle
    T = inps[0].X.shape[0]
    alpha = inps[0].alpha
    r = inps[0].A.shape[0]
    t_q = t_d = 0.0
    wds = []
    for inp in inps:
        n_out, n_in = inp.W.shape
        t0 = time.perf_counter()
        oc, oq, od = oracle.quantize_nf4(inp.W)
        t1 = time.perf_counter()
        wds.append(oracle.dequant(oc, oq, od, n_out, n_in))
        t_q += t1 - t0
        t_d += time.perf_counter() - t1
    passes = 2 if train else 1

    def run(ts):
        t0 = time.perf_counter()
        for inp, Wd in zip(inps, wds):
            oracle.linear_fwd(inp.X[:ts], Wd, inp.A, inp.B, alpha)
            if train:
                oracle.linear_bwd(inp.X[:ts], inp.dY[:ts], Wd, inp.A, inp.B, alpha)
        return time.perf_counter() - t0

    cap = max(1, min(T, slice_cap))
    ts = min(cap, 16)
    dt = run(ts)
    budget = max(2.0, target_s - t_q - t_d)
    ts = int(max(1, min(cap, ts * budget / max(dt, 1e-3))))
    dt = run(ts)
    reps = 1
    while dt < budget and ts == T:  # the whole batch is quicker than the target: repeat the pass
        dt += run(ts)
        reps += 1
    slice_s = dt / reps
    step_s = passes * t_d + slice_s * T / ts
    fl_step = sum(flops_linear(T, inp.W.shape[0], inp.W.shape[1], r, train) for inp in inps)
    kind = "fwd+bwd" if train else "fwd"
    return {"value": fl_step / step_s / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"quantize of all {len(inps)} weights in full ({t_q:.1f} s); {kind} of every linear on the "
                      f"first {ts} of {T} tokens ({reps} x {slice_s:.1f} s) plus one dequantization per pass "
                      f"({t_d:.1f} s per pass); binary64 C oracle, OpenMP"
                      + (f"; the full step's {step_s:.1f} s is extrapolated linearly in T" if ts < T else ""),
            "extrapolated": ts < T, "step_seconds": step_s, "quantize_seconds": t_q, "slice_tokens": ts,
            "slice_seconds": slice_s, "passes": reps}


def pct(xs, q):
    """q-th percentile (0..100) of a list, linear interpolation."""
    import numpy as np
    return float(np.percentile(np.asarray(xs, np.float64), q)) if xs else None


def launch_stats(times, per_step):
    """Per-launch times of one kernel (ms, launch order) split by their place in the step (one launch per
    linear per step): median, p10, p90 and average of each place."""
    out = []
    for i in range(per_step):
        xs = times[i::per_step]
        out.append({"launches": len(xs), "median_ms": pct(xs, 50), "p10_ms": pct(xs, 10), "p90_ms": pct(xs, 90),
                    "avg_ms": sum(xs) / len(xs) if xs else None})
    return out


def context_gemm(B, layers, T, train, steps, warmup):
    """Dense bf16 torch.mm (hipBLASLt) on the same shapes with each linear's dequantized weight stored as
    a dense bf16 matrix: X [T, K] . W'^T (forward) and dY [T, N] . W' (dX); no decode, no LoRA term.
    Both operands are contiguous row-major.  Context for the fused GEMMs only."""
    import torch
    dev = layers[0]["A"].device
    jobs = []
    for L in layers:
        W = B.dequant(L["copies"][0]["w"])
        Ws = [W, W.clone()]
        WTs = [w.t().contiguous() for w in Ws]
        c0 = L["copies"][0]
        Y = torch.empty((T, L["n_out"]), dtype=torch.bfloat16, device=dev)
        jobs.append(("fwd", L, c0["X"], WTs, Y, 2 * T * L["n_out"] * L["n_in"]))
        if train:
            dX = torch.empty((T, L["n_in"]), dtype=torch.bfloat16, device=dev)
            jobs.append(("dx", L, c0["dY"], Ws, dX, 2 * T * L["n_out"] * L["n_in"]))
    ev = {i: [] for i in range(len(jobs))}
    for it in range(warmup + steps):
        for i, (kind, L, A_, Bs, out, _) in enumerate(jobs):
            if it >= warmup:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                torch.mm(A_, Bs[it % 2], out=out)
                e1.record()
                ev[i].append((e0, e1))
            else:
                torch.mm(A_, Bs[it % 2], out=out)
    torch.cuda.synchronize()
    res = {"what": "torch.mm bf16 (hipBLASLt) on the same shapes, dense bf16 weight (no decode, no LoRA term), "
                   "median per launch over the timed steps", "per_linear": []}
    tot = {"fwd": [0.0, 0.0], "dx": [0.0, 0.0]}
    for i, (kind, L, *_, fl) in enumerate(jobs):
        ms = [a.elapsed_time(b) for a, b in ev[i]]
        med = pct(ms, 50)
        tot[kind][0] += fl
        tot[kind][1] += med
        res["per_linear"].append({"linear": L["name"], "pass": kind, "median_ms": med, "p10_ms": pct(ms, 10),
                                  "p90_ms": pct(ms, 90), "tflops": fl / (med * 1e-3) / 1e12})
    for kind, (fl, ms) in tot.items():
        if ms:
            res[kind + "_tflops"] = fl / (ms * 1e-3) / 1e12
            res[kind + "_frac_peak"] = res[kind + "_tflops"] / PEAK_BF16_TFLOPS
    return res


def flops_linear(T, N, K, r, train):
    f = 2 * T * N * K + 2 * T * r * (K + N)
    if train:
        f += 2 * T * N * K + 4 * T * r * (K + N)
    return f


def weight_bytes(N, K):
    nblk = N * K // 64
    return N * K // 2 + nblk + 4 * ((nblk + 255) // 256)


def bench_merge(args, B, layers, r, alpha):
    """Export merge of every linear: HBM bytes = NF4 weight read + bf16 merged weight written (+ A, B)."""
    import torch

    outs = [torch.empty((L["n_out"], L["n_in"]), dtype=torch.bfloat16, device=L["A"].device) for L in layers]

    def run(i):
        for L, o in zip(layers, outs):
            c = L["copies"][i % len(L["copies"])]
            st = c["w"].struct()
            B._check(B.load_library().qlora_merge(B.ctypes.byref(st), None, L["n_out"], L["n_in"], B._ptr(L["A"]),
                                                  B._ptr(L["B"]), r, float(alpha), B._ptr(o), None,
                                                  B._stream(o.device)), "qlora_merge")

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    B.timing_read("merge")
    B.timing_enable("merge", True)
    t0 = time.perf_counter()
    for i in range(args.steps):
        run(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    B.timing_enable("merge", False)
    n, ms = B.timing_read("merge")
    nbytes = sum(weight_bytes(L["n_out"], L["n_in"]) + 2 * L["n_out"] * L["n_in"] + 2 * r * (L["n_in"] + L["n_out"])
                 for L in layers)
    gbps = nbytes / (ms / args.steps * 1e-3) / 1e9
    traffic = traffic_from_profiles("merge", args.config + "_merge")
    print(json.dumps({"metric": "NF4 adapter merge for export, HBM GB/s", "value": gbps, "unit": "GB/s",
                      "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "ms_per_step": elapsed / args.steps * 1e3, "higher_is_better": True, "dtype": "bf16",
                      "data": "synthetic",
                      "config": {"workload": WORKLOAD_TEXT[args.config], "name": args.config + "_merge", "rank": r,
                                 "linears": [[L["name"], L["n_out"], L["n_in"]] for L in layers]},
                      "roofline": {"bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                   "frac": gbps / PEAK_HBM_GBPS,
                                   "traffic": traffic, "algorithmic_bytes_per_launch": nbytes / len(layers),
                                   "kernel": "merge",
                                   "avg_ms_per_launch": ms / n if n else None}}))


def bench_multi(args, B, layers, T, r, alpha, lins):
    """Forward of a batch cut into equal token segments, each with its own adapter of a pool."""
    import numpy as np
    import torch

    from bit_quantized_lora_02_amd.synth import linear_inputs

    S = args.adapters
    dev = layers[0]["A"].device
    bounds = [round(i * T / S) for i in range(S + 1)]
    seg = torch.tensor(bounds, dtype=torch.int32, device=dev)
    ad = torch.arange(S, dtype=torch.int32, device=dev)
    g = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    for li, L in enumerate(layers):
        pa, pb = [], []
        for i in range(S):
            inp = linear_inputs(L["n_out"], L["n_in"], 1, r, alpha, seed=500 + 31 * li + i, make_dy=False)
            pa.append(inp.A)
            pb.append(inp.B)
        L["A_pool"], L["B_pool"] = g(np.stack(pa)), g(np.stack(pb))
        L["ws_m"] = torch.empty(max(1, B.workspace_bytes(B.OP_FWD_MULTI, T, L["n_out"], L["n_in"], r)),
                                dtype=torch.uint8, device=dev)

    def step(i):
        for L in layers:
            c = L["copies"][i % len(L["copies"])]
            B.linear_fwd_multi(c["X"], c["w"], L["A_pool"], L["B_pool"], alpha, seg, ad, ws=L["ws_m"], out=c["Y"])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    timed = ["nf4_gemm_fwd", "nf4_gemv", "lora_u_multi"]
    t0 = time.perf_counter()  # wall clock without the per-kernel events, then a second pass with them
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    for k in timed:
        B.timing_read(k)
        B.timing_enable(k, True)
    for i in range(args.steps):
        step(args.steps + i)
    torch.cuda.synchronize()
    kernels = {}
    for k in timed:
        B.timing_enable(k, False)
        n, ms = B.timing_read(k)
        if n:
            kernels[k] = {"launches": n, "avg_ms_per_launch": ms / n, "ms_per_step": ms / args.steps}
    fl = sum(2 * T * L["n_out"] * L["n_in"] + 2 * T * r * (L["n_in"] + L["n_out"]) for L in layers)
    wb = sum(weight_bytes(L["n_out"], L["n_in"]) for L in layers)
    ms_step = elapsed / args.steps * 1e3
    print(json.dumps({"metric": "NF4 many-adapter forward TFLOP/s", "value": fl / (elapsed / args.steps) / 1e12,
                      "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "ms_per_step": ms_step, "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
                      "weight_stream_GBps": wb / (elapsed / args.steps) / 1e9,
                      "config": {"workload": WORKLOAD_TEXT[args.config].format(n=lins[0][1], t=T) +
                                 f", {S} adapters in {S} equal token segments", "tokens": T, "rank": r,
                                 "adapters": S, "linears": [[L["name"], L["n_out"], L["n_in"]] for L in layers]},
                      "kernels": kernels}))


def gpu_clocks():
    """Current GPU clocks as rocm-smi reports them (None where it is missing or fails)."""
    import shutil
    import subprocess
    exe = shutil.which("rocm-smi") or ("/opt/rocm/bin/rocm-smi" if os.path.exists("/opt/rocm/bin/rocm-smi") else None)
    if not exe:
        return None
    try:
        out = subprocess.run([exe, "--showclocks", "--json"], capture_output=True, text=True, timeout=20).stdout
        d = json.loads(out)
        card = next(iter(d.values()))
        return {k: v for k, v in card.items() if "clock" in k.lower() or k.lower().endswith("clk")} or card
    except Exception as e:  # a missing tool or a format change must not end the bench
        return {"error": str(e)[:200]}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this NF4 + LoRA linear runs on a single MI355X "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.traffic_from:  # post-processing of counter runs: no GPU needed
        lins, T, r, alpha, outliers, train = linears_for(args)
        wl = args.config if args.config != "small_token" else f"small_token_{lins[0][1]}x8192_T{T}"
        if args.merge:
            wl += "_merge"
        ks = [args.traffic_kernel] if args.traffic_kernel else ["merge"] if args.merge else (
            ["nf4_gemm_fwd", "nf4_gemm_dx"] if train else ["nf4_gemm_fwd", "nf4_gemv"])
        write_traffic(args, wl, ks)
        return

    import numpy as np
    import torch

    from bit_quantized_lora_02_amd import binding as B
    from bit_quantized_lora_02_amd.synth import linear_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calibrate_copy:
        nbytes = 256 << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": nbytes, "bytes_written": nbytes, "launches": 5}))
        return

    lins, T, r, alpha, outliers, train = linears_for(args)
    if args.steps <= 0:
        args.steps = 100 if train or T > 64 else 500
    drop = args.dropout
    if drop and (not train or not 0.0 < drop < 1.0):
        print("--dropout needs a training config and 0 < p < 1", file=sys.stderr)
        sys.exit(2)
    if args.copies <= 0:  # rotate through >= 512 MB so that a step does not find the previous one's lines cached
        per_copy = sum(weight_bytes(n, k) + 2 * T * (n + k) * (2 if train else 1) for _, n, k in lins)
        args.copies = int(min(32, max(2, -(-(512 << 20) // per_copy))))
    layers = []
    inps = []
    t_quant = 0.0
    for li, (name, n_out, n_in) in enumerate(lins):
        inp = linear_inputs(n_out, n_in, T, r, alpha, seed=li, outlier_frac=outliers, make_dy=train)
        inps.append(inp)
        Wg = torch.from_numpy(inp.W).to(dev)
        g = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        w = B.quantize_nf4(Wg)
        torch.cuda.synchronize()
        t_quant += time.perf_counter() - t0
        del Wg
        X, A, Bm = g(inp.X), g(inp.A), g(inp.B)
        dY = g(inp.dY) if train else None
        copies = []
        for c in range(max(1, args.copies)):
            wc = w if c == 0 else B.NF4Weight(w.n_out, w.n_in, w.codes.clone(), w.absmax_q.clone(),
                                              w.absmax_step.clone())
            copies.append(dict(w=wc, X=X if c == 0 else X.clone(), dY=(dY if c == 0 else dY.clone()) if train else None,
                               Y=torch.empty((T, n_out), dtype=torch.bfloat16, device=dev),
                               U=torch.empty((T, r), dtype=torch.bfloat16, device=dev),
                               dX=torch.empty((T, n_in), dtype=torch.bfloat16, device=dev) if train else None,
                               mask=torch.empty((T, n_in // 8), dtype=torch.uint8, device=dev) if drop else None))
        layers.append(dict(name=name, n_out=n_out, n_in=n_in, A=A, B=Bm, copies=copies,
                           dA=torch.empty_like(A), dB=torch.empty_like(Bm),
                           adam=[B.AdamState.zeros_like(A), B.AdamState.zeros_like(Bm)] if args.adamw else None,
                           adam8=[B.Adam8State.zeros_like(A), B.Adam8State.zeros_like(Bm)] if args.adamw8 else None,
                           ws_f=torch.empty(max(1, B.workspace_bytes(B.OP_FWD_DROPOUT if drop else B.OP_FWD, T,
                                                                     n_out, n_in, r)), dtype=torch.uint8, device=dev),
                           ws_b=torch.empty(max(1, B.workspace_bytes(B.OP_BWD, T, n_out, n_in, r)), dtype=torch.uint8,
                                            device=dev) if train else None))

    if args.merge:
        bench_merge(args, B, layers, r, alpha)
        return
    if args.adapters:
        bench_multi(args, B, layers, T, r, alpha, lins)
        return

    def step(i):
        step_layers(i)
        if args.adamw and train:  # one launch updates every adapter matrix of the step
            B.adamw_step([t for L in layers for t in (L["A"], L["B"])], [t for L in layers for t in (L["dA"], L["dB"])],
                         [s_ for L in layers for s_ in L["adam"]], lr=2e-4, step=i + 1)
        if args.adamw8 and train:
            B.adamw8_step([t for L in layers for t in (L["A"], L["B"])],
                          [t for L in layers for t in (L["dA"], L["dB"])], [s_ for L in layers for s_ in L["adam8"]],
                          lr=2e-4, step=i + 1)

    def step_layers(i):
        for L in layers:
            c = L["copies"][i % len(L["copies"])]
            if drop:  # a fresh mask per step: the step index is the generator offset
                B.linear_fwd_dropout(c["X"], c["w"], L["A"], L["B"], alpha, drop, seed=2024, offset=i, ws=L["ws_f"],
                                     out=c["Y"], u_out=c["U"], mask_out=c["mask"])
                B.linear_bwd_dropout(c["X"], c["dY"], c["w"], L["A"], L["B"], alpha, drop, c["mask"], U=c["U"],
                                     ws=L["ws_b"], outs=(c["dX"], L["dA"], L["dB"]))
                continue
            B.linear_fwd(c["X"], c["w"], L["A"], L["B"], alpha, ws=L["ws_f"], out=c["Y"], u_out=c["U"])
            if train:
                B.linear_bwd(c["X"], c["dY"], c["w"], L["A"], L["B"], alpha, U=c["U"], ws=L["ws_b"],
                             outs=(c["dX"], L["dA"], L["dB"]))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    timed = ["nf4_gemm_fwd", "nf4_gemm_dx"] if train else ["nf4_gemm_fwd", "nf4_gemv"]
    if args.adamw and train:
        timed.append("adamw")
    if args.adamw8 and train:
        timed.append("adamw8")
    # the wall-clock steps run without the per-kernel events (a launch that carries them costs the host
    # about 25 us more, which would make the microsecond-scale small-token step host-bound) ...
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # ... and the same steps once more with them, for the per-kernel times
    for k in timed:
        B.timing_read(k)  # clear
        B.timing_enable(k, True)
    for i in range(args.steps):
        step(args.steps + i)
    torch.cuda.synchronize()
    for k in timed:
        B.timing_enable(k, False)
    each = {k: B.timing_read_each(k, cap=1 << 20) for k in timed}
    ktimes = {k: (len(v), sum(v)) for k, v in each.items()}

    ms_step = elapsed / args.steps * 1e3
    fl_step = sum(flops_linear(T, L["n_out"], L["n_in"], r, train) for L in layers)
    wb_step = sum(weight_bytes(L["n_out"], L["n_in"]) for L in layers) * (2 if train else 1)
    tflops = fl_step / (elapsed / args.steps) / 1e12
    wgbps = wb_step / (elapsed / args.steps) / 1e9

    # per-kernel algorithmic work per launch, summed over the layers of one step
    kflops = {
        "nf4_gemm_fwd": sum(2 * T * L["n_out"] * (L["n_in"] + r) for L in layers),
        "nf4_gemm_dx": sum(2 * T * L["n_in"] * (L["n_out"] + r) for L in layers),
        "nf4_gemv": sum(2 * T * L["n_out"] * L["n_in"] for L in layers),
        "adamw": 0,
        "adamw8": 0,
    }
    kbytes = {  # compulsory HBM bytes of one launch: weight stream + activations in and out + LoRA operands
        "nf4_gemm_fwd": sum(weight_bytes(L["n_out"], L["n_in"]) + 2 * T * (L["n_in"] + L["n_out"]) +
                            2 * (T + L["n_out"]) * r for L in layers),
        "nf4_gemm_dx": sum(weight_bytes(L["n_out"], L["n_in"]) + 2 * T * (L["n_in"] + L["n_out"]) +
                           2 * (T + L["n_in"]) * r for L in layers),
        # the small-token kernel reads the weight stream and X; its binary32 partials are not algorithmic
        "nf4_gemv": sum(weight_bytes(L["n_out"], L["n_in"]) + 2 * T * L["n_in"] for L in layers),
        # per adapter element: bf16 param and grad read, param written; binary32 m and v read and written
        "adamw": sum(22 * r * (L["n_in"] + L["n_out"]) for L in layers),
        # bf16 param and grad read, param written; one code of each moment read and written (+ absmax)
        "adamw8": sum(10 * r * (L["n_in"] + L["n_out"]) for L in layers),
    }
    kernels = {}
    for k, (n, ms) in ktimes.items():
        if n == 0:
            continue
        per_step_launches = n / args.steps if args.steps else 0
        avg_ms = ms / n if n else float("nan")
        kernels[k] = {"launches": n, "avg_ms_per_launch": avg_ms,
                      "ms_per_step": ms / args.steps,
                      "tflops": kflops[k] / (ms / args.steps * 1e-3) / 1e12 if ms and kflops[k] else None,
                      "gbps": kbytes[k] / (ms / args.steps * 1e-3) / 1e9 if ms else None,
                      "launches_per_step": per_step_launches}
        if per_step_launches == len(layers):  # one launch per linear per step: statistics per linear
            st = launch_stats(each[k], len(layers))
            med_step = sum(x["median_ms"] for x in st)
            kernels[k]["per_linear"] = [dict(linear=L["name"], **x) for L, x in zip(layers, st)]
            kernels[k]["median_ms_per_step"] = med_step
            kernels[k]["tflops_median"] = kflops[k] / (med_step * 1e-3) / 1e12 if kflops[k] else None
            kernels[k]["gbps_median"] = kbytes[k] / (med_step * 1e-3) / 1e9
    dom = max((k for k in kernels if k not in ("adamw", "adamw8")), key=lambda k: kernels[k]["ms_per_step"])
    kd = kernels[dom]
    wl = args.config if args.config != "small_token" else f"small_token_{lins[0][1]}x8192_T{T}"
    if drop:
        wl += f"_dropout{drop:g}"
    traffic = traffic_from_profiles(dom, wl)
    if train or T > 80:
        roof = {"bound": "mfma", "achieved": kd["tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": kd["tflops"] / PEAK_BF16_TFLOPS, "traffic": traffic, "kernel": dom,
                "avg_ms_per_launch": kd["avg_ms_per_launch"]}
        if "tflops_median" in kd:
            roof["achieved_median"] = kd["tflops_median"]
            roof["frac_median"] = kd["tflops_median"] / PEAK_BF16_TFLOPS
    else:
        roof = {"bound": "hbm", "achieved": kd["gbps"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": kd["gbps"] / PEAK_HBM_GBPS, "traffic": traffic, "kernel": dom,
                "avg_ms_per_launch": kd["avg_ms_per_launch"]}
        if "gbps_median" in kd:
            roof["achieved_median"] = kd["gbps_median"]
            roof["frac_median"] = kd["gbps_median"] / PEAK_HBM_GBPS
    roof["algorithmic_per_step"] = kflops[dom] if roof["bound"] == "mfma" else kbytes[dom]

    ctx = None
    if not args.no_context_gemm and (train or T > 64):
        log("timing the dense bf16 context GEMMs ...")
        ctx = context_gemm(B, layers, T, train, min(args.steps, 100), 10)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(inps, train, args.cpu_seconds,
                           128 if args.config in ("mlp_8b", "layer_70b") else T)

    text = WORKLOAD_TEXT[args.config].format(n=lins[0][1], t=T)
    if drop:
        text += f", LoRA dropout p={drop:g}"
    line = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": text, "name": wl, "tokens": T, "rank": r, "alpha": alpha,
                   "pass": ("fwd+bwd+adamw" if args.adamw else "fwd+bwd+adamw8" if args.adamw8 else "fwd+bwd")
                   if train else "fwd", "lora_dropout": drop,
                   "linears": [[L["name"], L["n_out"], L["n_in"]] for L in layers],
                   "parallelism": "single GPU"},
        "weight_stream_GBps": wgbps,
        "weight_stream_frac_hbm": wgbps / PEAK_HBM_GBPS,
        "quantize_ms": t_quant * 1e3,
        "rotating_copies": args.copies,
        "roofline": roof,
        "kernels": kernels,
        "context_gemm": ctx,
        "clocks": gpu_clocks(),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
