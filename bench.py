"""Benchmark of the SS1 linear-layer forward on one MI355X.

One step = one ss1_forward call (input sketch, contraction, epilogue: the whole
hot path) over one batch of synthetic inputs already resident in HBM.  By
default the workload is the GPT-2 Small MLP up-projection at 2x compression
(M=8192 tokens, K=768, N=3072, c=2, BK=64, BN=64, bf16).  Steps rotate through
enough distinct input/output buffer sets (> 512 MB in total, twice the MALL)
that every step reads its operands from HBM, not from a warm cache.

Prints ONE JSON line: dense-equivalent TFLOP/s (2*M*N*K per step / time), the
fraction of the binding roofline of the dominant kernel (MFMA bf16 on the
compressed FLOPs 2*M*N*K/c, or HBM on the algorithmic bytes
e*(M*K + N*K/c + M*N), whichever bound is the larger lower time), and the CPU
oracle timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--workload gpt2s_up]
                    [--algo auto] [--index] [--warm] [--no-cpu-baseline]
                    [--sweep FILE]   # one extra JSON line per workload into FILE
    python bench.py --copy-calibration   # a plain 256 MiB device copy, for counters
    python bench.py --op project [--workload llama_gateup_m1]
        # ss1_project instead: least-squares projection of the layer's dense
        # [N][K] weight onto its sharing pattern, GB/s against the HBM roofline

roofline.traffic is the HBM traffic of one launch measured with rocprofv3
FETCH_SIZE and WRITE_SIZE counters, each scaled by what the counter reads for
the plain copy of --copy-calibration; it is read from
profiles/traffic_counters.json and reported only while the kernel source the
counters were taken on is unchanged (else null).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SS1 layer dense-equiv TFLOP/s + % of MFMA/HBM roofline at M×K×N, c"
PEAK_MFMA_BF16 = 2.5e15     # MI355X dense bf16 MFMA, FLOP/s
PEAK_MFMA_F32 = 157.3e12
PEAK_HBM = 8.0e12           # MI355X HBM3E, B/s
HEADLINE = "gpt2s_up"
SWEEP = ["gpt2s_up", "gpt2l_up", "gpt2l_down", "llama_gateup_m1", "llama_down_m1",
         "llama_gateup_m16", "llama_down_m16", "llama_gateup_m4096", "llama_down_m4096"] + [
    f"square_c{c}_bn{bn}" for c in (1, 2, 4, 8) for bn in (32, 64, 128)]
PROJECT_HEADLINE = "llama_gateup_m1"   # the Llama-3-8B gate/up weight, 14336 x 4096
PROJECT_SWEEP = ["llama_gateup_m1", "llama_down_m1", "gpt2s_up", "gpt2l_up"]


def work(wl):
    e = 2 if wl.dtype == "bf16" else 4
    return {
        "dense_flops": 2 * wl.M * wl.N * wl.K,
        "compressed_flops": 2 * wl.M * wl.N * wl.K // wl.c,
        "bytes": e * (wl.M * wl.K + wl.N * wl.Kc + wl.M * wl.N) + wl.G * wl.J * 5,
        "sketch_adds": wl.G * wl.M * wl.Kc * (wl.c - 1),
        "x_l2_bytes": e * wl.G * wl.M * wl.K,
    }


def roofline(wl, t):
    """Roofline record of one launch lasting t seconds."""
    wk = work(wl)
    peak_f = PEAK_MFMA_BF16 if wl.dtype == "bf16" else PEAK_MFMA_F32
    t_f = wk["compressed_flops"] / peak_f
    t_b = wk["bytes"] / PEAK_HBM
    mf = {"achieved": wk["compressed_flops"] / t / 1e12, "peak": peak_f / 1e12, "unit": "TFLOP/s"}
    hb = {"achieved": wk["bytes"] / t / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    mf["frac"] = mf["achieved"] / mf["peak"]
    hb["frac"] = hb["achieved"] / hb["peak"]
    if t_f >= t_b:
        r = {"bound": "mfma", **mf, "other": {"bound": "hbm", **hb}}
    else:
        r = {"bound": "hbm", **hb, "other": {"bound": "mfma", **mf}}
    r["t_lower_us"] = max(t_f, t_b) * 1e6
    traffic = recorded_traffic(wl.name)
    r["traffic"] = traffic
    r["traffic_unit"] = "HBM bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE)"
    r["traffic_vs_algorithmic"] = (traffic / wk["bytes"]) if traffic else None
    return r


CSRC = os.path.join(ROOT, "sketched_parameter_sharing_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def kernel_source_sha256():
    """Hash of every device source (kernels and the headers they include)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def recorded_traffic(name):
    """Calibrated HBM bytes per launch for record `name` (a workload, or
    "project:<workload>") from the committed counter record, or None when
    there is none or the kernels changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    w = rec.get("workloads", {}).get(name)
    if not w:
        return None
    return w.get("hbm_bytes_per_launch")


def copy_calibration(n=20):
    """A plain device copy of 256 MiB, repeated n times: the known-size
    reference for the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    nbytes = 256 << 20
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(n):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "copies": n}))


def to_dev(a, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def time_gpu(wl, steps, warmup, algo, use_index, warm):
    """Returns (seconds per step, kernel name, number of buffer sets)."""
    import torch
    import sketched_parameter_sharing_amd as ss1
    from ss1_inputs import make_inputs

    inp = make_inputs(wl)
    plan = ss1.DevicePlan.make(wl.plan_seed, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    e = 2 if wl.dtype == "bf16" else 4
    set_bytes = e * (wl.M * wl.K + wl.N * wl.Kc + wl.M * wl.N)
    nsets = 1 if warm else max(2, int(np.ceil(512e6 / max(set_bytes, 1))) + 1)
    nsets = min(nsets, 64)
    x0 = to_dev(inp.x_bits if wl.dtype == "bf16" else inp.x, wl.dtype)
    w0 = to_dev(inp.w_bits if wl.dtype == "bf16" else inp.w, wl.dtype)
    xs = [x0] + [x0.clone() for _ in range(nsets - 1)]
    ws = [w0] + [w0.clone() for _ in range(nsets - 1)]
    ys = [torch.empty((wl.M, wl.N), dtype=x0.dtype, device="cuda") for _ in range(nsets)]

    def step(i):
        k = i % nsets
        plan.forward(xs[k], ws[k], y=ys[k], algo=algo, use_index=use_index)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    t = start.elapsed_time(end) / 1e3 / steps
    return t, nsets


def project_work(wl):
    e = 2 if wl.dtype == "bf16" else 4
    return {"bytes": e * (wl.N * wl.K + wl.N * wl.Kc) + wl.G * wl.J * 5,
            "adds": wl.N * wl.Kc * (wl.c - 1)}


def time_project(wl, steps, warmup, warm):
    """ss1_project over rotating weight sets: (seconds per call, sets)."""
    import torch
    import sketched_parameter_sharing_amd as ss1
    from ss1_inputs import make_dense_weight

    vals, bits = make_dense_weight(wl)
    plan = ss1.DevicePlan.make(wl.plan_seed, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    set_bytes = project_work(wl)["bytes"]
    nsets = 1 if warm else min(64, max(2, int(np.ceil(512e6 / set_bytes)) + 1))
    W0 = to_dev(bits if wl.dtype == "bf16" else vals, wl.dtype)
    Ws = [W0] + [W0.clone() for _ in range(nsets - 1)]
    Cs = [torch.empty((wl.N, wl.Kc), dtype=W0.dtype, device="cuda") for _ in range(nsets)]

    def step(i):
        k = i % nsets
        ss1.project(Ws[k], plan.hash, plan.sign, wl.c, wl.BK, wl.BN, W_c=Cs[k])

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3 / steps, nsets


def cpu_baseline_project(wl, budget_s=10.0):
    """The oracle's projection, float64, on a bounded sample of groups."""
    import oracle
    from ss1_inputs import make_dense_weight

    cores = len(os.sched_getaffinity(0))
    h, s = oracle.plan(wl.plan_seed, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    vals, _ = make_dense_weight(wl)
    vals = vals.astype(np.float64)
    e = 2 if wl.dtype == "bf16" else 4
    ng, t, reps = 1, 0.0, 0
    while True:
        rows = ng * wl.BN
        t0 = time.perf_counter()
        oracle.project(vals[:rows], h[:ng], s[:ng], wl.K, rows, wl.c, wl.BK, wl.BN)
        t = time.perf_counter() - t0
        reps += 1
        if t > budget_s / 4 or ng >= wl.G:
            break
        ng = min(wl.G, ng * 4)
    nbytes = e * rows * (wl.K + wl.Kc)
    return {"value": nbytes / t / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{ng} of {wl.G} groups ({rows} of {wl.N} rows) of the {wl.name} weight, "
                      f"float64 NumPy oracle (single-threaded loops), {t:.3f} s "
                      f"(the sample's algorithmic bytes / time)"}


def kernel_name(wl, algo):
    """The kernel a call runs: the requested one, or what the library picks."""
    if algo != "auto":
        return algo
    import sketched_parameter_sharing_amd as ss1
    return ss1.select_algo(wl.M, wl.K, wl.N, wl.c, wl.BK, wl.BN, wl.dtype)


def cpu_baseline(wl, budget_s=10.0):
    """The oracle as it stands, float64, on a bounded sample of rows."""
    import oracle
    from ss1_inputs import make_inputs

    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        nt = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
        if nt:
            cores = max(nt)
    except Exception:
        pass
    h, s = oracle.plan(wl.plan_seed, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    rows = min(wl.M, 256)
    inp = make_inputs(wl.with_m(rows))
    t0 = time.perf_counter()
    oracle.forward(inp.x, inp.w, h, s, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    t1 = time.perf_counter() - t0
    # scale the sample to about budget_s of CPU time
    rows = int(min(wl.M, max(rows, rows * budget_s / max(t1, 1e-3))))
    inp = make_inputs(wl.with_m(rows))
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.forward(inp.x, inp.w, h, s, wl.K, wl.N, wl.c, wl.BK, wl.BN)
        reps += 1
        if time.perf_counter() - t0 > budget_s or reps >= 3:
            break
    t = (time.perf_counter() - t0) / reps
    return {"value": 2 * rows * wl.N * wl.K / t / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{rows} of {wl.M} rows of {wl.name}, float64 NumPy oracle, {reps} rep(s), "
                      f"{t:.3f} s each (dense-equivalent FLOPs of the sample / time)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None,
                    help=f"default: {HEADLINE} (forward), {PROJECT_HEADLINE} (project)")
    ap.add_argument("--op", default="forward", choices=["forward", "project"])
    ap.add_argument("--algo", default="auto", choices=["auto", "fused", "smallm", "generic", "band"])
    ap.add_argument("--index", action="store_true", help="time ss1_forward_idx (inverse index plan)")
    ap.add_argument("--warm", action="store_true", help="reuse one buffer set (cache-warm)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", default=None, help="also time every workload, JSON lines into this file")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 256 MiB device copy (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build runs on a single MI355X and has no "
              "multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import sketched_parameter_sharing_amd as ss1
    from ss1_inputs import WORKLOADS
    ss1.load()

    def measure(name, steps, warmup):
        wl = WORKLOADS[name]
        t, nsets = time_gpu(wl, steps, warmup, args.algo, args.index, args.warm)
        wk = work(wl)
        rec = {
            "metric": METRIC,
            "value": wk["dense_flops"] / t / 1e12,
            "unit": "TFLOP/s",
            "n_gpus": 1,
            "steps": steps,
            "warmup": warmup,
            "ms_per_step": t * 1e3,
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": wl.dtype,
            "data": "synthetic (seeded N(0,1) inputs, N(0,0.02) compressed weights, seeded balanced plan)",
            "config": {"workload": name, "M": wl.M, "K": wl.K, "N": wl.N, "c": wl.c, "BK": wl.BK,
                       "BN": wl.BN, "kernel": kernel_name(wl, args.algo),
                       "plan": "inverse index" if args.index else "hash",
                       "cache": "warm" if args.warm else f"cold ({nsets} rotating buffer sets)",
                       "compressed_tflops": wk["compressed_flops"] / t / 1e12,
                       "x_l2_gb": wk["x_l2_bytes"] / 1e9},
            "roofline": roofline(wl, t),
        }
        return rec, wl

    def measure_project(name, steps, warmup):
        wl = WORKLOADS[name]
        t, nsets = time_project(wl, steps, warmup, args.warm)
        wk = project_work(wl)
        traffic = recorded_traffic("project:" + name)
        rec = {
            "metric": "SS1 weight projection GB/s (dense [N][K] read + compressed [N][K/c] written) "
                      "+ % of HBM roofline",
            "value": wk["bytes"] / t / 1e9,
            "unit": "GB/s",
            "n_gpus": 1,
            "steps": steps,
            "warmup": warmup,
            "ms_per_step": t * 1e3,
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": wl.dtype,
            "data": "synthetic (seeded N(0,0.02) dense weight, seeded balanced plan)",
            "config": {"workload": name + "_weight_projection", "N": wl.N, "K": wl.K, "c": wl.c,
                       "BK": wl.BK, "BN": wl.BN, "kernel": "project",
                       "cache": "warm" if args.warm else f"cold ({nsets} rotating buffer sets)"},
            "roofline": {"bound": "hbm", "achieved": wk["bytes"] / t / 1e9, "peak": PEAK_HBM / 1e9,
                         "unit": "GB/s", "frac": wk["bytes"] / t / PEAK_HBM, "traffic": traffic,
                         "traffic_unit": "HBM bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE)",
                         "traffic_vs_algorithmic": (traffic / wk["bytes"]) if traffic else None,
                         "t_lower_us": wk["bytes"] / PEAK_HBM * 1e6},
        }
        return rec, wl

    if args.sweep:
        with open(args.sweep, "w") as f:
            for name in SWEEP:
                rec, _ = measure(name, max(20, args.steps // 4), max(5, args.warmup // 4))
                f.write(json.dumps(rec) + "\n")
                print(f"sweep {name}: {rec['ms_per_step'] * 1e3:.1f} us, "
                      f"{rec['roofline']['bound']} frac {rec['roofline']['frac']:.3f}",
                      file=sys.stderr, flush=True)
            for name in PROJECT_SWEEP:
                rec, _ = measure_project(name, max(20, args.steps // 4), max(5, args.warmup // 4))
                f.write(json.dumps(rec) + "\n")
                print(f"sweep project {name}: {rec['ms_per_step'] * 1e3:.1f} us, "
                      f"hbm frac {rec['roofline']['frac']:.3f}", file=sys.stderr, flush=True)

    if args.op == "project":
        name = args.workload or PROJECT_HEADLINE
        rec, wl = measure_project(name, args.steps, args.warmup)
        rec["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_project(wl)
        print(json.dumps(rec), flush=True)
        return

    rec, wl = measure(args.workload or HEADLINE, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
