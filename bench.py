"""Benchmark of the SS1 linear-layer forward on one MI355X.

One step = one ss1_forward call (input sketch, contraction, epilogue: the whole
hot path) over one batch of synthetic inputs already resident in HBM.  By
default the workload is the largest single-GPU configuration, the
Llama-3-8B-shaped gate/up projection at 2x compression (M=4096 tokens,
K=4096, N=14336, c=2, BK=64, BN=64, bf16).  Steps rotate through enough
distinct input/output buffer sets (> 512 MB in total, twice the MALL) that
every step reads its operands from HBM, not from a warm cache.  The K timed
steps run as at least 20 trials of equal length, each bracketed by events on
the stream the library launches on; ms_per_step is the median trial's time
per step (p10 / p90 beside it), the whole region is also timed.

Prints ONE JSON line: dense-equivalent TFLOP/s (2*M*N*K per step / time), the
fraction of the binding roofline of the dominant kernel (MFMA bf16 on the
compressed FLOPs 2*M*N*K/c, or HBM on the algorithmic bytes
e*(M*K + N*K/c + M*N), whichever bound is the larger lower time) against the
spec peak and against the peak measured by the probes of --peaks, the L2
operand traffic of the fold kernel against the measured L2-to-LDS rate, and
the CPU oracle (float64, and float32) timed on a bounded sample of the same
workload.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--workload llama_gateup_m4096]
                    [--algo auto] [--index] [--warm] [--graph] [--no-cpu-baseline]
                    [--sweep FILE]   # one extra JSON line per workload into FILE
        # --graph: the timed calls captured in one HIP graph and replayed
        # (forward and fp8 ops), so no host launch cost falls in the timed
        # region; the microsecond decode layers otherwise time the host too
    python bench.py --copy-calibration   # a plain 256 MiB device copy, for counters
    python bench.py --op mlp [--mlp-c 4] [--row-chunk 8192]
        # ss1_mlp_forward: the GPT-2 L MLP pair (8192 x 1280 -> 5120 -> 1280,
        # GELU between) at compression c, with a c sweep against the dense
        # pair (torch bf16 matmuls and GELU at the same shapes)
    python bench.py --op backward [--workload gpt2s_up]
        # ss1_backward (dx and dW_c) of the layer, next to the dense layer's
        # two backward GEMMs (torch bf16) at the same shapes
    python bench.py --op fp8 [--workload llama_gateup_m1]
        # ss1_forward_fp8w: the layer with per-row fp8 (E4M3) compressed
        # weights, against the HBM / MFMA roofline on its own bytes
    python bench.py --op project [--workload llama_gateup_m1]
        # ss1_project instead: least-squares projection of the layer's dense
        # [N][K] weight onto its sharing pattern, GB/s against the HBM roofline

roofline.traffic is the HBM traffic of one step measured with rocprofv3
counters (reads from TCC_EA0_RDREQ / _128B / _32B, writes from WRITE_SIZE),
checked against the plain copy of --copy-calibration; it is read from
profiles/traffic_counters.json and reported only while the kernel sources the
counters were taken on are unchanged (else null).
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
HEADLINE = "llama_gateup_m4096"
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


def fold_operand_bytes(wl, cus):
    """Bytes the fold kernel moves from L2 into LDS per call (the x tile and
    the expanded weight tile of every stage of every tile), for its usual
    256 x 256 tiles: when they end in a partial round of compute units, the
    neurons past the last whole round run as 128 x 256 tiles (the library's
    split launch); 192 x 256 tiles where those fill one round of tiles with
    fewer tile rows (GPT-2 L down).  A model of the launch, not a counter."""
    M, N, K = wl.M, wl.N, wl.K
    e = 2
    if N % 256:
        return None
    n_mt, n_nt = -(-M // 256), N // 256
    tiles = n_mt * n_nt
    full = tiles // cus
    main = N
    if full and tiles % cus:
        n_main = full * cus // n_mt
        if 0 < n_main < n_nt:
            single = -(-tiles // cus)
            split = -(-(n_mt * n_main) // cus) + 0.55 * -(-((-(-M // 128)) * (n_nt - n_main)) // cus)
            if split < 0.97 * single:
                main = n_main * 256
    cost256 = 256 * (-(-(n_mt * (main // 256)) // cus) + (0.55 * -(-((-(-M // 128)) * ((N - main) // 256)) // cus)
                                                         if main != N else 0))
    cost192 = 192 * -(-((-(-M // 192)) * n_nt) // cus)
    if cost192 < cost256:
        return (-(-M // 192)) * n_nt * K * (192 + 256) * e
    b = n_mt * (main // 256) * K * (256 + 256) * e
    if main != N:
        b += (-(-M // 128)) * ((N - main) // 256) * K * (128 + 256) * e
    return b


def roofline(wl, t, kernel=None, peaks=None):
    """Roofline record of one launch lasting t seconds of `kernel`; with
    `peaks` (measured_peaks()), the fraction of the measured peak too and, for
    the fold kernel, its L2-to-LDS operand traffic against the measured
    buffer-to-LDS rate."""
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
    if peaks:
        meas = (peaks["mfma_bf16_tflops"] * 1e12 if r["bound"] == "mfma" else peaks["hbm_read_tbs"] * 1e12)
        unit_div = 1e12 if r["bound"] == "mfma" else 1e9
        r["measured_peak"] = {"peak": meas / unit_div, "unit": r["unit"], "frac": r["achieved"] / (meas / unit_div),
                              "source": "bench.py --peaks probes, same process"}
        if kernel == "fold":
            import torch
            cus = torch.cuda.get_device_properties(0).multi_processor_count
            ob = fold_operand_bytes(wl, cus)
            if ob:
                r["l2_operand"] = {"bytes": ob, "achieved_tbs": ob / t / 1e12,
                                   "peak_tbs": peaks["l2_dma_tbs"], "frac": ob / t / 1e12 / peaks["l2_dma_tbs"],
                                   "note": "x and expanded-weight tiles moved L2 -> LDS per call (tile model) "
                                           "against the measured buffer-to-LDS read rate"}
    # a record per workload for the kernel auto picks, "<family>:<workload>" for the others
    traffic = recorded_traffic(wl.name, kernel) or recorded_traffic(f"{kernel}:{wl.name}", kernel)
    r["traffic"] = traffic
    r["traffic_unit"] = "HBM bytes per step (TCC_EA0_RDREQ* read bytes + WRITE_SIZE; all launches of one call)"
    r["traffic_vs_algorithmic"] = (traffic / wk["bytes"]) if traffic else None
    return r


CSRC = os.path.join(ROOT, "sketched_parameter_sharing_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


# Device sources of each kernel family (its kernels and the headers they include).
KERNEL_SOURCES = {
    "band": ("ss1_kernels.hip", "ss1_device.h", "ss1_internal.h", "ss1_msketch.h"),
    "fused": ("ss1_kernels.hip", "ss1_device.h", "ss1_internal.h"),
    "smallm": ("ss1_kernels.hip", "ss1_device.h", "ss1_internal.h"),
    "gemv": ("ss1_gemv.hip", "ss1_device.h", "ss1_internal.h"),
    "decode": ("ss1_decode.hip", "ss1_device.h", "ss1_dma.h", "ss1_internal.h"),
    "split": ("ss1_decode.hip", "ss1_device.h", "ss1_dma.h", "ss1_internal.h"),
    "generic": ("ss1_kernels.hip", "ss1_device.h", "ss1_internal.h"),
    "fold": ("ss1_fold.hip", "ss1_device.h", "ss1_dma.h", "ss1_internal.h"),
    "fold8": ("ss1_fold.hip", "ss1_quant.hip", "ss1_device.h", "ss1_dma.h", "ss1_internal.h"),
    "project": ("ss1_project.hip", "ss1_device.h", "ss1_internal.h"),
    "group": ("ss1_group.hip", "ss1_device.h", "ss1_dma.h", "ss1_internal.h", "ss1_msketch.h"),
}


def kernel_family(kernel_name):
    """Family of a kernel from its (demangled or short) name, e.g.
    'void band_kernel<...>' -> 'band'."""
    for fam in KERNEL_SOURCES:
        if f"{fam}_kernel" in kernel_name:
            return fam
    return None


def kernel_source_sha256(names=None):
    """Hash of the given device sources (default: every kernel source and
    header)."""
    if names is None:
        names = [n for n in os.listdir(CSRC) if n.endswith((".hip", ".h"))]
    h = hashlib.sha256()
    for name in sorted(names):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def recorded_traffic(name, kernel=None):
    """HBM bytes per step (every launch of one call) for record `name` (a
    workload, or "project:<workload>" / "fp8:<workload>") from the committed
    counter record, or None when there is none, when it measured another
    kernel family than `kernel`, or when the sources of its kernels changed
    since."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    w = rec.get("records", {}).get(name)
    if not w or "sources" not in w:
        return None
    if kernel is not None and w.get("family") != kernel:
        return None
    if w.get("sources_sha256") != kernel_source_sha256(w["sources"]):
        return None
    return w.get("hbm_bytes_per_step")


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


def measured_peaks():
    """Measured machine rates from the probes of libss1_peaks.so, each timed
    with events over one launch on the current stream:
      mfma_bf16_tflops  16x16x32 bf16 MFMA issue rate, 8 chains per wave
      l2_read_tbs       reads into registers of a 2 MiB window every block
                        shares (L2-resident after the first sweep)
      l2_dma_tbs        the same window by direct buffer-to-LDS loads, 1 KB
                        of consecutive bytes per wave-load
      l2_dma_half_tbs   buffer-to-LDS loads of 64-byte half rows, one per
                        128-byte line (a 32-column bf16 tile of a matrix)
      hbm_read_tbs      reads of a 4 GiB buffer, each block its own 2 MiB
      hbm_copy_tbs      torch's device copy of 1 GiB (read + write bytes)
      lds_read_tbs      ds_read_b128 at conflict-free addresses, immediate
                        offsets (few vector instructions per read)
      lds_read_valu_addr_tbs  the same reads with every address computed in
                        the loop"""
    import ctypes
    import torch
    here = os.path.join(ROOT, "sketched_parameter_sharing_amd", "libss1_peaks.so")
    lib = ctypes.CDLL(here)
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream or None
    vp = ctypes.c_void_p

    def timed(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        best = None
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            t = a.elapsed_time(b) / 1e3
            best = t if best is None else min(best, t)
        return best

    out = {}
    blocks, iters = 256 * 8, 4096
    t = timed(lambda: lib.ss1_peak_mfma(blocks, iters, vp(sink.data_ptr()), vp(st)))
    out["mfma_bf16_tflops"] = blocks * 4 * iters * 8 * 2 * 16 * 16 * 32 / t / 1e12
    win, reps, nb = 2 << 20, 16, 2048
    buf = torch.zeros(4 << 30, dtype=torch.uint8, device="cuda")
    t = timed(lambda: lib.ss1_peak_read(nb, vp(buf.data_ptr()), ctypes.c_uint32(win), reps, 0,
                                        vp(sink.data_ptr()), vp(st)))
    out["l2_read_tbs"] = nb * reps * win / t / 1e12
    t = timed(lambda: lib.ss1_peak_dma(nb, 256, vp(buf.data_ptr()), ctypes.c_uint32(win), reps, 0,
                                       vp(sink.data_ptr()), vp(st)))
    out["l2_dma_tbs"] = nb * reps * win / t / 1e12
    t = timed(lambda: lib.ss1_peak_dma(nb, 256, vp(buf.data_ptr()), ctypes.c_uint32(win), reps, 1,
                                       vp(sink.data_ptr()), vp(st)))
    out["l2_dma_half_tbs"] = nb * reps * win / 2 / t / 1e12
    hwin = 2 << 20
    nh = (4 << 30) // hwin
    t = timed(lambda: lib.ss1_peak_read(nh, vp(buf.data_ptr()), ctypes.c_uint32(hwin), 1, 1,
                                        vp(sink.data_ptr()), vp(st)))
    out["hbm_read_tbs"] = nh * hwin / t / 1e12
    src = buf[: 1 << 30]
    dst = buf[2 << 30: (2 << 30) + (1 << 30)]
    t = timed(lambda: dst.copy_(src))
    out["hbm_copy_tbs"] = 2 * (1 << 30) / t / 1e12
    li = 2048
    t = timed(lambda: lib.ss1_peak_lds(256 * 8, li, 1, vp(sink.data_ptr()), vp(st)))
    out["lds_read_tbs"] = 256 * 8 * 256 * li * 8 * 16 / t / 1e12
    t = timed(lambda: lib.ss1_peak_lds(256 * 8, li, 0, vp(sink.data_ptr()), vp(st)))
    out["lds_read_valu_addr_tbs"] = 256 * 8 * 256 * li * 8 * 16 / t / 1e12
    del buf
    return out


def to_dev(a, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def time_graph(fn, steps, warmup):
    """Seconds per call of fn(i), i < steps, captured in one HIP graph and
    replayed: the launches cost no host time in the timed region."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(warmup):
            fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3 / steps


def time_gpu(wl, steps, warmup, algo, use_index, warm, graph=False):
    """Returns (seconds per step, number of buffer sets)."""
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
    # the auto path goes through ss1_forward_ws: a workspace (allocated here,
    # outside the timed region) lets decode shapes whose input rows are too
    # long for the decode kernel split each group's columns over blocks; for
    # every other shape it runs as ss1_forward and the workspace is unused
    work = None
    if algo == "auto" and not use_index:
        _, nbytes = ss1.forward_ws_query(wl.M, wl.K, wl.N, wl.c, wl.BK, wl.BN,
                                         ss1.BF16 if wl.dtype == "bf16" else ss1.F32)
        if nbytes:
            work = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def step(i):
        k = i % nsets
        if work is not None:
            ss1.forward_ws(xs[k], ws[k], plan.hash, plan.sign, wl.c, wl.BK, wl.BN, workspace=work, y=ys[k])
        else:
            plan.forward(xs[k], ws[k], y=ys[k], algo=algo, use_index=use_index)

    if graph:
        t = time_graph(step, steps, warmup)
        return t, nsets, {"median": t, "p10": t, "p90": t, "mean": t, "trials": 1, "steps_per_trial": steps}
    for i in range(warmup):
        step(i)
    stats = time_trials(step, steps)
    return stats["median"], nsets, stats


def time_dense_layer(wl, steps, warmup, warm=False):
    """The dense layer of the same shape, y = x @ W^T with W [N][K] (torch's
    GEMM, hipBLASLt on ROCm), cold over rotating buffer sets as time_gpu
    rotates the SS1 layer's: seconds per step (median over trials)."""
    import torch
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    e = 2 if wl.dtype == "bf16" else 4
    set_bytes = e * (wl.M * wl.K + wl.N * wl.K + wl.M * wl.N)
    nsets = 1 if warm else min(64, max(2, int(np.ceil(512e6 / max(set_bytes, 1))) + 1))
    g = torch.Generator(device="cuda").manual_seed(7)
    xs = [torch.randn(wl.M, wl.K, device="cuda", dtype=dt, generator=g) for _ in range(nsets)]
    ws = [(0.02 * torch.randn(wl.N, wl.K, device="cuda", dtype=torch.float32, generator=g)).to(dt)
          for _ in range(nsets)]
    ys = [torch.empty(wl.M, wl.N, device="cuda", dtype=dt) for _ in range(nsets)]

    def step(i):
        k = i % nsets
        torch.mm(xs[k], ws[k].t(), out=ys[k])

    for i in range(warmup):
        step(i)
    return time_trials(step, steps)["median"]


def time_trials(step, steps, min_trials=20):
    """Times exactly `steps` calls of step(i) as at least `min_trials` trials
    of equal length (the last one takes the remainder), each bracketed by
    events recorded on the current stream, the one the library launches on;
    the whole region is bracketed by synchronizations.  Returns seconds per
    step: median, p10, p90 over trials, and the mean over the whole region."""
    import torch
    per = max(1, steps // min_trials)
    bounds = list(range(0, steps, per)) + [steps]
    ev = [torch.cuda.Event(enable_timing=True) for _ in bounds]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    for b in range(len(bounds) - 1):
        for i in range(bounds[b], bounds[b + 1]):
            step(i)
        ev[b + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step = np.array([ev[b].elapsed_time(ev[b + 1]) / 1e3 / (bounds[b + 1] - bounds[b])
                         for b in range(len(bounds) - 1)])
    total = ev[0].elapsed_time(ev[-1]) / 1e3
    return {"median": float(np.median(per_step)), "p10": float(np.percentile(per_step, 10)),
            "p90": float(np.percentile(per_step, 90)), "mean": total / steps, "trials": len(per_step),
            "steps_per_trial": per, "wall_s": wall}


def project_work(wl):
    e = 2 if wl.dtype == "bf16" else 4
    return {"bytes": e * (wl.N * wl.K + wl.N * wl.Kc) + wl.G * wl.J * 5,
            "adds": wl.N * wl.Kc * (wl.c - 1)}


def fp8_work(wl):
    return {"dense_flops": 2 * wl.M * wl.N * wl.K, "compressed_flops": 2 * wl.M * wl.N * wl.K // wl.c,
            "bytes": 2 * wl.M * wl.K + wl.N * wl.Kc + 4 * wl.N + 2 * wl.M * wl.N + wl.G * wl.J * 5}


def time_fp8(wl, steps, warmup, warm, graph=False):
    """ss1_forward_fp8w over rotating buffer sets: (seconds per call, sets)."""
    import torch
    import sketched_parameter_sharing_amd as ss1
    from ss1_inputs import make_inputs

    inp = make_inputs(wl)
    plan = ss1.DevicePlan.make(wl.plan_seed, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    Q0, s0 = ss1.quantize_fp8(to_dev(inp.w_bits, "bf16"))
    set_bytes = fp8_work(wl)["bytes"]
    nsets = 1 if warm else min(64, max(2, int(np.ceil(512e6 / set_bytes)) + 1))
    x0 = to_dev(inp.x_bits, "bf16")
    xs = [x0] + [x0.clone() for _ in range(nsets - 1)]
    Qs = [Q0] + [Q0.clone() for _ in range(nsets - 1)]
    Ss = [s0] + [s0.clone() for _ in range(nsets - 1)]
    ys = [torch.empty((wl.M, wl.N), dtype=x0.dtype, device="cuda") for _ in range(nsets)]

    def step(i):
        k = i % nsets
        ss1.forward_fp8w(xs[k], Qs[k], Ss[k], plan.hash, plan.sign, wl.c, wl.BK, wl.BN, y=ys[k])

    if graph:
        return time_graph(step, steps, warmup), nsets
    return time_events_i(step, steps, warmup), nsets


def fp8a_work(wl):
    """Per step: quantize x (read bf16, write E4M3 codes and row scales), then
    the fp8 layer (read the codes, W_c codes and scales, write bf16 y)."""
    return {"dense_flops": 2 * wl.M * wl.N * wl.K, "compressed_flops": 2 * wl.M * wl.N * wl.K // wl.c,
            "bytes": 2 * wl.M * wl.K + (wl.M * wl.K + 4 * wl.M) * 2 + wl.N * wl.Kc + 4 * wl.N + 2 * wl.M * wl.N
                     + wl.G * wl.J * 5}


def time_fp8a(wl, steps, warmup):
    """One step = ss1_quantize_fp8 of x then ss1_forward_fp8 (W_c quantized
    once, as weights are), over rotating buffer sets: returns
    (seconds per step, sets, seconds of the forward alone)."""
    import torch
    import sketched_parameter_sharing_amd as ss1
    from ss1_inputs import make_inputs

    inp = make_inputs(wl)
    plan = ss1.DevicePlan.make(wl.plan_seed, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    Q, ws = ss1.quantize_fp8(to_dev(inp.w_bits, "bf16"))
    nsets = min(64, max(2, int(np.ceil(512e6 / fp8a_work(wl)["bytes"])) + 1))
    x0 = to_dev(inp.x_bits, "bf16")
    xs = [x0] + [x0.clone() for _ in range(nsets - 1)]
    xq = [torch.empty(x0.shape, dtype=torch.uint8, device="cuda") for _ in range(nsets)]
    sc = [torch.empty((wl.M,), dtype=torch.float32, device="cuda") for _ in range(nsets)]
    ys = [torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device="cuda") for _ in range(nsets)]

    def step(i):
        k = i % nsets
        ss1.quantize_fp8(xs[k], Q=xq[k], scale=sc[k])
        ss1.forward_fp8(xq[k], sc[k], Q, ws, plan.hash, plan.sign, wl.c, wl.BK, wl.BN, y=ys[k])

    def fwd(i):
        k = i % nsets
        ss1.forward_fp8(xq[k], sc[k], Q, ws, plan.hash, plan.sign, wl.c, wl.BK, wl.BN, y=ys[k])

    t = time_events_i(step, steps, warmup)
    t_fwd = time_events_i(fwd, steps, warmup)
    return t, nsets, t_fwd


def time_events_i(fn, steps, warmup):
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3 / steps


def backward_work(wl):
    dw = 2 * wl.M * wl.N * wl.Kc          # dy_g^T z_g per group
    dx = 2 * wl.M * wl.N * wl.K           # dy times the dense expansion
    return {"flops": dw + dx, "dense_equiv_flops": 2 * 2 * wl.M * wl.N * wl.K,
            "bytes": 2 * (2 * wl.M * wl.K + 2 * wl.N * wl.Kc + wl.M * wl.N)}


def time_backward(wl, steps, warmup, warm=False):
    """ss1_backward (dx and dW_c) per call, and the dense layer's two backward
    GEMMs at the same shapes; cold (default): rotating sets of every operand
    and output totalling over 512 MB.  Returns (seconds, dense seconds, sets)."""
    import torch
    import sketched_parameter_sharing_amd as ss1
    from ss1_inputs import make_inputs, draw, f32_to_bf16_bits
    inp = make_inputs(wl)
    p = ss1.DevicePlan.make(wl.plan_seed, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    x0, w0 = to_dev(inp.x_bits, "bf16"), to_dev(inp.w_bits, "bf16")
    dy0 = to_dev(f32_to_bf16_bits(draw("normal", wl.x_seed + 7, (wl.M, wl.N))), "bf16")
    set_bytes = 2 * (2 * wl.M * wl.K + 2 * wl.N * wl.Kc + wl.M * wl.N)
    nsets = 1 if warm else min(16, max(2, int(np.ceil(512e6 / set_bytes)) + 1))
    sets = [(x0, w0, dy0)] + [(x0.clone(), w0.clone(), dy0.clone()) for _ in range(nsets - 1)]
    outs = [(torch.empty_like(x0), torch.empty_like(w0)) for _ in range(nsets)]

    def step(i):
        x, w, dy = sets[i % nsets]
        dx, dw = outs[i % nsets]
        ss1.backward(x, w, p.hash, p.sign, wl.c, wl.BK, wl.BN, dy, dx=dx, dW_c=dw)

    t = time_events_i(step, steps, warmup)
    # the dense layer's backward at the same shapes: dx = dy W, dW = dy^T x
    W0 = to_dev(f32_to_bf16_bits(draw("normal002", wl.w_seed, (wl.N, wl.K))), "bf16")
    dsets = [(dy, dy.t().contiguous(), x, W0 if k == 0 else W0.clone()) for k, (x, _, dy) in enumerate(sets)]

    def dense(i):
        dy, dyt, x, W = dsets[i % nsets]
        torch.matmul(dy, W)
        torch.matmul(dyt, x)

    t_dense = time_events_i(dense, steps, warmup)
    return t, t_dense, nsets


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
    reps, t0 = 0, time.perf_counter()   # repeat the largest sample to about budget_s
    while True:
        oracle.project(vals[:rows], h[:ng], s[:ng], wl.K, rows, wl.c, wl.BK, wl.BN)
        reps += 1
        if time.perf_counter() - t0 > budget_s or reps >= 100:
            break
    t = (time.perf_counter() - t0) / reps
    nbytes = e * rows * (wl.K + wl.Kc)
    return {"value": nbytes / t / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{ng} of {wl.G} groups ({rows} of {wl.N} rows) of the {wl.name} weight, "
                      f"float64 NumPy oracle (single-threaded loops), {reps} rep(s) of {t:.3f} s "
                      f"(the sample's algorithmic bytes / time)"}


MLP_SHAPE = {"M": 8192, "K": 1280, "N1": 5120, "N2": 1280, "BK": 64, "BN": 64}  # GPT-2 L MLP pair


def mlp_work(c, m=MLP_SHAPE):
    M, K, N1, N2 = m["M"], m["K"], m["N1"], m["N2"]
    dense = 2 * M * K * N1 + 2 * M * N1 * N2
    return {"dense_flops": dense, "compressed_flops": dense // c,
            "bytes": 2 * (M * K + N1 * K // c + N2 * N1 // c + M * N2)}


def mlp_bk(c, m=MLP_SHAPE):
    """Chunk width of the pair at compression c: 64, or 32 where K/64 chunks
    do not split into c equal parts (c = 8 at K = 1280)."""
    return m["BK"] if (m["K"] // m["BK"]) % c == 0 else m["BK"] // 2


def mlp_kernel_families(c, row_chunk, m=MLP_SHAPE):
    """The kernels ss1_mlp_forward runs for the pair's up and down layers at
    chunks of row_chunk rows (ss1_select_algo)."""
    import sketched_parameter_sharing_amd as ss1
    R, BK, BN = min(row_chunk, m["M"]), mlp_bk(c, m), m["BN"]
    return (ss1.select_algo(R, m["K"], m["N1"], c, BK, BN, "bf16"),
            ss1.select_algo(R, m["N1"], m["N2"], c, BK, BN, "bf16"))


def mlp_recorded_traffic(c, row_chunk):
    """The pair's recorded HBM bytes per call, or None when the record's kernels
    are not the ones the pair runs now or their sources changed since."""
    name = f"mlp:gpt2l_mlp_pair_c{c}_r{row_chunk}"
    try:
        with open(TRAFFIC_FILE) as f:
            w = json.load(f).get("records", {}).get(name)
    except (OSError, ValueError):
        return None
    if not w or "sources" not in w:
        return None
    fams = set(mlp_kernel_families(c, row_chunk))
    if {kernel_family(k["kernel"]) for k in w.get("kernels", [])} != fams:
        return None
    if not all(set(KERNEL_SOURCES[f]) <= set(w["sources"]) for f in fams):
        return None
    return recorded_traffic(name)


def make_mlp(c, m=MLP_SHAPE, seed=0x5f00):
    """Device tensors of an SS1 MLP pair at compression c (seeded inputs)."""
    import torch
    import sketched_parameter_sharing_amd as ss1
    from ss1_inputs import draw, f32_to_bf16_bits
    M, K, N1, N2, BK, BN = m["M"], m["K"], m["N1"], m["N2"], mlp_bk(c, m), m["BN"]
    x = to_dev(f32_to_bf16_bits(draw("normal", seed, (M, K))), "bf16")
    layers = []
    for i, (k, n) in enumerate(((K, N1), (N1, N2))):
        s = seed + 1 + i + 16 * c
        w = to_dev(f32_to_bf16_bits(draw("normal002", s, (n, k // c))), "bf16")
        p = ss1.DevicePlan.make(s, k, n, c, BK, BN)
        layers.append((w, p.hash, p.sign, c, BK, BN))
    return x, layers[0], layers[1]


def time_events(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3 / steps


def time_mlp(c, steps, warmup, row_chunk, warm=False):
    """ss1_mlp_forward per call; cold (default): rotating sets of x, both
    weights, h and y totalling over 512 MB, so every call reads its operands
    from HBM.  Returns (seconds per call, sets)."""
    import torch
    import sketched_parameter_sharing_amd as ss1
    x0, up0, down0 = make_mlp(c)
    R = min(row_chunk, x0.shape[0])
    set_bytes = 2 * (x0.numel() + up0[0].numel() + down0[0].numel() + R * up0[0].shape[0]
                     + x0.shape[0] * down0[0].shape[0])
    nsets = 1 if warm else min(16, max(2, int(np.ceil(512e6 / set_bytes)) + 1))
    sets = []
    for k in range(nsets):
        x = x0 if k == 0 else x0.clone()
        up = up0 if k == 0 else (up0[0].clone(),) + tuple(up0[1:])
        down = down0 if k == 0 else (down0[0].clone(),) + tuple(down0[1:])
        h = torch.empty((R, up0[0].shape[0]), dtype=x0.dtype, device="cuda")
        y = torch.empty((x0.shape[0], down0[0].shape[0]), dtype=x0.dtype, device="cuda")
        sets.append((x, up, down, h, y))

    def step(i):
        x, up, down, h, y = sets[i % nsets]
        ss1.mlp_forward(x, up, down, h=h, y=y)

    return time_events_i(step, steps, warmup), nsets


def time_dense_mlp(steps, warmup, m=MLP_SHAPE, warm=False):
    """The dense pair at the same shapes: torch (hipBLASLt) bf16 matmuls and
    torch's erf GELU, weights [out][in] as a linear layer's; cold (default)
    over rotating sets of x, both weights and y like time_mlp."""
    import torch
    from ss1_inputs import draw, f32_to_bf16_bits
    M, K, N1, N2 = m["M"], m["K"], m["N1"], m["N2"]
    x = to_dev(f32_to_bf16_bits(draw("normal", 0x5f00, (M, K))), "bf16")
    w1 = to_dev(f32_to_bf16_bits(draw("normal002", 0x5f01, (N1, K))), "bf16")
    w2 = to_dev(f32_to_bf16_bits(draw("normal002", 0x5f02, (N2, N1))), "bf16")
    w1t, w2t = w1.t().contiguous(), w2.t().contiguous()
    set_bytes = 2 * (M * K + 2 * N1 * K + M * N1 + M * N2)
    nsets = 1 if warm else min(16, max(2, int(np.ceil(512e6 / set_bytes)) + 1))
    sets = [(x, w1t, w2t)] + [(x.clone(), w1t.clone(), w2t.clone()) for _ in range(nsets - 1)]
    gelu = torch.nn.GELU()

    def step(i):
        a, b, c = sets[i % nsets]
        torch.matmul(gelu(torch.matmul(a, b)), c)

    return time_events_i(step, steps, warmup)


def cpu_baseline_mlp(c, budget_s=10.0, m=MLP_SHAPE):
    """The oracle's MLP pair, float64, on a bounded sample of rows."""
    import oracle
    from ss1_inputs import draw, f32_to_bf16_bits, bf16_bits_to_f32
    K, N1, N2, BK, BN = m["K"], m["N1"], m["N2"], mlp_bk(c, m), m["BN"]

    def layer(k, n, s):
        w = bf16_bits_to_f32(f32_to_bf16_bits(draw("normal002", s, (n, k // c)))).astype(np.float64)
        h, sg = oracle.plan(s, k, n, c, BK, BN)
        return {"Wc": w, "hash": h, "sign": sg, "K": k, "N": n, "c": c, "BK": BK, "BN": BN}

    up, down = layer(K, N1, 0x5f00 + 1 + 16 * c), layer(N1, N2, 0x5f00 + 2 + 16 * c)
    rows, t = 16, 0.0
    while True:
        x = draw("normal", 0x5f00, (rows, K)).astype(np.float64)
        t0 = time.perf_counter()
        oracle.mlp_forward(x, up, down)
        t = time.perf_counter() - t0
        if t > budget_s / 3 or rows >= m["M"]:
            break
        rows = min(m["M"], rows * 4)
    flops = mlp_work(c, dict(m, M=rows))["dense_flops"]
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        nt = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
        if nt:
            cores = max(nt)
    except Exception:
        pass
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{rows} of {m['M']} rows of the GPT-2 L MLP pair at c={c}, float64 NumPy oracle, "
                      f"{t:.3f} s (dense-equivalent FLOPs of the sample / time)"}


def fp8_kernel_name(wl):
    """The kernel ss1_forward_fp8w runs for this layer (the library's choice)."""
    import sketched_parameter_sharing_amd as ss1
    return ss1.select_algo(wl.M, wl.K, wl.N, wl.c, wl.BK, wl.BN, wl.dtype, weights="fp8")


def kernel_name(wl, algo):
    """The kernel a call runs: the requested one, or what the library picks
    for ss1_forward_ws (the auto path; it equals ss1_forward's choice except
    where the column-split decode with a workspace applies)."""
    if algo != "auto":
        return algo
    import sketched_parameter_sharing_amd as ss1
    return ss1.forward_ws_query(wl.M, wl.K, wl.N, wl.c, wl.BK, wl.BN,
                                ss1.BF16 if wl.dtype == "bf16" else ss1.F32)[0]


def cpu_baseline(wl, budget_s=10.0):
    """The oracle as it stands, float64 (its definition) and float32 (the
    same steps, for CPU speed), each on a bounded sample of rows."""
    r64 = cpu_baseline_dtype(wl, np.float64, budget_s)
    r32 = cpu_baseline_dtype(wl, np.float32, budget_s)
    r64["float32"] = {"value": r32["value"], "unit": r32["unit"], "sample": r32["sample"]}
    return r64


def cpu_baseline_dtype(wl, dtype, budget_s=10.0):
    """The oracle's forward in `dtype` on a bounded sample of rows."""
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
    name = np.dtype(dtype).name
    t0 = time.perf_counter()
    oracle.forward(inp.x, inp.w, h, s, wl.K, wl.N, wl.c, wl.BK, wl.BN, dtype=dtype)
    t1 = time.perf_counter() - t0
    # scale the sample to about budget_s of CPU time
    rows = int(min(wl.M, max(rows, rows * budget_s / max(t1, 1e-3))))
    inp = make_inputs(wl.with_m(rows))
    reps = 0
    t0 = time.perf_counter()
    while True:   # whole-workload samples repeat until about budget_s of CPU time
        oracle.forward(inp.x, inp.w, h, s, wl.K, wl.N, wl.c, wl.BK, wl.BN, dtype=dtype)
        reps += 1
        if time.perf_counter() - t0 > budget_s or reps >= 50:
            break
    t = (time.perf_counter() - t0) / reps
    return {"value": 2 * rows * wl.N * wl.K / t / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{rows} of {wl.M} rows of {wl.name}, {name} NumPy oracle, {reps} rep(s), "
                      f"{t:.3f} s each (dense-equivalent FLOPs of the sample / time)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None,
                    help=f"default: {HEADLINE} (forward), {PROJECT_HEADLINE} (project)")
    ap.add_argument("--op", default="forward", choices=["forward", "project", "mlp", "fp8", "fp8a", "backward"])
    ap.add_argument("--mlp-c", type=int, default=4, help="compression of the timed MLP pair (op mlp)")
    ap.add_argument("--row-chunk", type=int, default=8192, help="rows per chunk of the MLP pair (op mlp)")
    ap.add_argument("--mlp-only", action="store_true",
                    help="op mlp: time only the pair at --mlp-c and --row-chunk and the dense pair (for profiling)")
    ap.add_argument("--algo", default="auto", choices=["auto", "fused", "smallm", "gemv", "decode", "generic", "band", "fold", "group"])
    ap.add_argument("--index", action="store_true", help="time ss1_forward_idx (inverse index plan)")
    ap.add_argument("--warm", action="store_true", help="reuse one buffer set (cache-warm)")
    ap.add_argument("--graph", action="store_true",
                    help="capture the timed calls in one HIP graph (forward and fp8 ops): no host launch "
                         "cost in the timed region, for microsecond decode layers")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip timing the dense layer of the same shape beside the forward")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the machine-rate probes (roofline against spec peaks only); for profiler runs")
    ap.add_argument("--sweep", default=None, help="also time every workload, JSON lines into this file")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 256 MiB device copy (counter calibration)")
    ap.add_argument("--peaks", action="store_true",
                    help="run only the machine-rate probes (MFMA, L2, LDS-DMA, HBM, LDS) and print them")
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
    if args.peaks:
        print(json.dumps({"measured_peaks": measured_peaks()}), flush=True)
        return
    import sketched_parameter_sharing_amd as ss1
    from ss1_inputs import WORKLOADS
    ss1.load()

    peaks = None if (args.no_peaks or args.op != "forward") else measured_peaks()

    def measure(name, steps, warmup):
        wl = WORKLOADS[name]
        t, nsets, stats = time_gpu(wl, steps, warmup, args.algo, args.index, args.warm, args.graph)
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
                       "launch": "one HIP graph of the timed calls" if args.graph else "eager",
                       "compressed_tflops": wk["compressed_flops"] / t / 1e12,
                       "x_l2_gb": wk["x_l2_bytes"] / 1e9,
                       "timing": {"trials": stats["trials"], "steps_per_trial": stats["steps_per_trial"],
                                  "ms_per_step_median": stats["median"] * 1e3,
                                  "ms_per_step_p10": stats["p10"] * 1e3, "ms_per_step_p90": stats["p90"] * 1e3,
                                  "ms_per_step_mean": stats["mean"] * 1e3}},
        }
        rec["roofline"] = roofline(wl, t, rec["config"]["kernel"], peaks)
        if peaks:
            rec["config"]["measured_peaks"] = peaks
        if rec["config"]["kernel"] == "fold":
            # the fold kernel multiplies by the expanded weight: its matrix
            # cores execute the dense FLOP count, c times the algorithmic one
            rec["config"]["executed_mfma_tflops"] = wk["dense_flops"] / t / 1e12
        if not args.no_dense:
            td = time_dense_layer(wl, max(20, steps // 2), max(5, warmup // 2), args.warm)
            rec["config"]["dense_layer_ms"] = td * 1e3
            rec["config"]["speedup_vs_dense_layer"] = td / t
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
                         "traffic_unit": "HBM bytes per call (TCC_EA0_RDREQ* read bytes + WRITE_SIZE)",
                         "traffic_vs_algorithmic": (traffic / wk["bytes"]) if traffic else None,
                         "t_lower_us": wk["bytes"] / PEAK_HBM * 1e6},
        }
        return rec, wl

    def sweep_steps(wl):
        # at least ~2 ms of timed work (the roofline time taken twice), so the
        # start of the timed region does not weigh on microsecond layers
        wk = work(wl)
        t_low = max(wk["compressed_flops"] / PEAK_MFMA_BF16, wk["bytes"] / PEAK_HBM)
        return max(20, args.steps // 4, min(1000, int(np.ceil(2e-3 / (2 * t_low)))))

    if args.sweep:
        with open(args.sweep, "w") as f:
            for name in SWEEP:
                rec, _ = measure(name, sweep_steps(WORKLOADS[name]), max(5, args.warmup // 4))
                f.write(json.dumps(rec) + "\n")
                print(f"sweep {name}: {rec['ms_per_step'] * 1e3:.1f} us, "
                      f"{rec['roofline']['bound']} frac {rec['roofline']['frac']:.3f}",
                      file=sys.stderr, flush=True)
            for name in PROJECT_SWEEP:
                rec, _ = measure_project(name, max(20, args.steps // 4), max(5, args.warmup // 4))
                f.write(json.dumps(rec) + "\n")
                print(f"sweep project {name}: {rec['ms_per_step'] * 1e3:.1f} us, "
                      f"hbm frac {rec['roofline']['frac']:.3f}", file=sys.stderr, flush=True)

    if args.op == "mlp":
        c = args.mlp_c
        t, nsets = time_mlp(c, args.steps, args.warmup, args.row_chunk, args.warm)
        wk = mlp_work(c)
        t_dense = time_dense_mlp(max(20, args.steps // 2), max(5, args.warmup // 2), warm=args.warm)
        sweep = []
        for cc in ((c,) if args.mlp_only else (2, 4, 8)):
            tc = t if cc == c else time_mlp(cc, max(20, args.steps // 2), max(5, args.warmup // 2), args.row_chunk,
                                            args.warm)[0]
            sweep.append({"c": cc, "BK": mlp_bk(cc), "ms": tc * 1e3, "dense_equiv_tflops": mlp_work(cc)["dense_flops"] / tc / 1e12,
                          "speedup_vs_dense": t_dense / tc})
        chunks = []
        for R in (() if args.mlp_only else (8192, 4096, 2048, 1024)):
            if R == args.row_chunk:
                continue
            tr = time_mlp(c, max(20, args.steps // 2), max(5, args.warmup // 2), R, args.warm)[0]
            chunks.append({"row_chunk": R, "ms": tr * 1e3})
        t_f = wk["compressed_flops"] / PEAK_MFMA_BF16
        t_b = wk["bytes"] / PEAK_HBM
        mf = {"bound": "mfma", "achieved": wk["compressed_flops"] / t / 1e12, "peak": PEAK_MFMA_BF16 / 1e12,
              "unit": "TFLOP/s"}
        hb = {"bound": "hbm", "achieved": wk["bytes"] / t / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
        for r in (mf, hb):
            r["frac"] = r["achieved"] / r["peak"]
        roof = dict(mf if t_f >= t_b else hb)
        roof["other"] = hb if t_f >= t_b else mf
        roof.update({"traffic": mlp_recorded_traffic(c, args.row_chunk),
                     "t_lower_us": max(t_f, t_b) * 1e6,
                     "note": "whole pair (both projections and the GELU epilogue) per call"})
        roof["traffic_vs_algorithmic"] = roof["traffic"] / wk["bytes"] if roof["traffic"] else None
        rec = {
            "metric": "SS1 MLP pair (up, GELU, down) dense-equiv TFLOP/s + % of MFMA/HBM roofline",
            "value": wk["dense_flops"] / t / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": t * 1e3, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) inputs, N(0,0.02) compressed weights, seeded balanced plans)",
            "config": {"workload": f"gpt2l_mlp_pair_c{c}", **MLP_SHAPE, "BK": mlp_bk(c), "c": c,
                       "row_chunk": args.row_chunk,
                       "cache": "warm (one buffer set)" if args.warm else f"cold ({nsets} rotating buffer sets)",
                       "dense_pair_ms": t_dense * 1e3, "speedup_vs_dense": t_dense / t, "c_sweep": sweep,
                       "row_chunk_sweep": chunks},
            "roofline": roof,
        }
        rec["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_mlp(c)
        print(json.dumps(rec), flush=True)
        return

    if args.op == "backward":
        name = args.workload or HEADLINE
        wl = WORKLOADS[name]
        t, t_dense, nsets = time_backward(wl, args.steps, args.warmup, args.warm)
        wk = backward_work(wl)
        mf = {"bound": "mfma", "achieved": wk["flops"] / t / 1e12, "peak": PEAK_MFMA_BF16 / 1e12,
              "unit": "TFLOP/s"}
        mf["frac"] = mf["achieved"] / mf["peak"]
        hb = {"bound": "hbm", "achieved": wk["bytes"] / t / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
        hb["frac"] = hb["achieved"] / hb["peak"]
        t_f, t_b = wk["flops"] / PEAK_MFMA_BF16, wk["bytes"] / PEAK_HBM
        roof = dict(mf if t_f >= t_b else hb)
        traffic = recorded_traffic("backward:" + name, "fold")
        roof.update({"other": hb if t_f >= t_b else mf, "traffic": traffic, "t_lower_us": max(t_f, t_b) * 1e6,
                     "traffic_vs_algorithmic": traffic / wk["bytes"] if traffic else None,
                     "note": "dx (dense-cost GEMM on the expanded weight) plus dW_c, both kernels per call"})
        rec = {
            "metric": "SS1 layer backward (dx + dW_c) TFLOP/s + % of MFMA/HBM roofline",
            "value": wk["flops"] / t / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": t * 1e3, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) inputs and upstream gradient, N(0,0.02) weights, seeded plan)",
            "config": {"workload": name + "_backward", "M": wl.M, "K": wl.K, "N": wl.N, "c": wl.c,
                       "BK": wl.BK, "BN": wl.BN,
                       "cache": "warm (one buffer set)" if args.warm else f"cold ({nsets} rotating buffer sets)",
                       "dense_backward_ms": t_dense * 1e3, "ratio_to_dense": t / t_dense},
            "roofline": roof,
        }
        if args.no_cpu_baseline:
            rec["cpu_baseline"] = None
        else:
            import oracle
            from ss1_inputs import make_inputs, draw
            rows = 64
            sub = wl.with_m(rows)
            inp = make_inputs(sub)
            h, sg = oracle.plan(wl.plan_seed, wl.K, wl.N, wl.c, wl.BK, wl.BN)
            dyh = draw("normal", 1, (rows, wl.N)).astype(np.float64)
            t0 = time.perf_counter()
            oracle.backward(inp.x, inp.w, dyh, h, sg, wl.K, wl.N, wl.c, wl.BK, wl.BN)
            tc = time.perf_counter() - t0
            rec["cpu_baseline"] = {"value": backward_work(sub)["flops"] / tc / 1e12, "unit": "TFLOP/s",
                                   "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
                                   "sample": f"{rows} of {wl.M} rows of {name}, float64 NumPy oracle backward, "
                                             f"{tc:.3f} s"}
        print(json.dumps(rec), flush=True)
        return

    if args.op == "fp8":
        name = args.workload or "llama_gateup_m1"
        wl = WORKLOADS[name]
        t, nsets = time_fp8(wl, args.steps, args.warmup, args.warm, args.graph)
        t16, _, _ = time_gpu(wl, max(20, args.steps // 2), max(5, args.warmup // 2), "auto", False, args.warm,
                          args.graph)
        wk = fp8_work(wl)
        t_f = wk["compressed_flops"] / PEAK_MFMA_BF16
        t_b = wk["bytes"] / PEAK_HBM
        mf = {"bound": "mfma", "achieved": wk["compressed_flops"] / t / 1e12, "peak": PEAK_MFMA_BF16 / 1e12,
              "unit": "TFLOP/s"}
        hb = {"bound": "hbm", "achieved": wk["bytes"] / t / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
        for r in (mf, hb):
            r["frac"] = r["achieved"] / r["peak"]
        roof = dict(mf if t_f >= t_b else hb)
        roof["other"] = hb if t_f >= t_b else mf
        traffic = recorded_traffic("fp8:" + name)
        roof.update({"traffic": traffic, "t_lower_us": max(t_f, t_b) * 1e6,
                     "traffic_vs_algorithmic": (traffic / wk["bytes"]) if traffic else None})
        rec = {
            "metric": "SS1 layer with fp8 (E4M3) weights: dense-equiv TFLOP/s + % of MFMA/HBM roofline",
            "value": wk["dense_flops"] / t / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": t * 1e3, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16 activations, fp8 e4m3 weights",
            "data": "synthetic (seeded N(0,1) inputs, N(0,0.02) compressed weights quantized per row, "
                    "seeded balanced plan)",
            "config": {"workload": name + "_fp8w", "M": wl.M, "K": wl.K, "N": wl.N, "c": wl.c, "BK": wl.BK,
                       "BN": wl.BN, "kernel": fp8_kernel_name(wl),
                       "cache": "warm" if args.warm else f"cold ({nsets} rotating buffer sets)",
                       "launch": "one HIP graph of the timed calls" if args.graph else "eager",
                       "bf16_weights_ms": t16 * 1e3, "speedup_vs_bf16_weights": t16 / t},
            "roofline": roof,
        }
        if args.no_cpu_baseline:
            rec["cpu_baseline"] = None
        else:
            rec["cpu_baseline"] = cpu_baseline(wl)
            rec["cpu_baseline"]["sample"] += " (bf16-weight oracle: the fp8 layer's arithmetic is the same)"
        print(json.dumps(rec), flush=True)
        return

    if args.op == "fp8a":
        name = args.workload or HEADLINE
        wl = WORKLOADS[name]
        t, nsets, t_fwd = time_fp8a(wl, args.steps, args.warmup)
        t16, _, _ = time_gpu(wl, max(20, args.steps // 2), max(5, args.warmup // 2), "auto", False, False)
        wk = fp8a_work(wl)
        peak8 = 5.0e15   # MI355X dense fp8 MFMA
        mf = {"bound": "mfma", "achieved": wk["compressed_flops"] / t / 1e12, "peak": peak8 / 1e12,
              "unit": "TFLOP/s"}
        mf["frac"] = mf["achieved"] / mf["peak"]
        hb = {"bound": "hbm", "achieved": wk["bytes"] / t / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
        hb["frac"] = hb["achieved"] / hb["peak"]
        t_f, t_b = wk["compressed_flops"] / peak8, wk["bytes"] / PEAK_HBM
        roof = dict(mf if t_f >= t_b else hb)
        roof.update({"other": hb if t_f >= t_b else mf, "traffic": recorded_traffic("fp8a:" + name, "fold8"),
                     "traffic_vs_algorithmic": None,
                     "t_lower_us": max(t_f, t_b) * 1e6,
                     "note": "per step: x quantized to E4M3 per row, then the fp8 fold (dense fp8 MFMA work "
                             "2*M*N*K; the compressed count is the algorithmic one)"})
        if roof["traffic"]:
            roof["traffic_vs_algorithmic"] = roof["traffic"] / wk["bytes"]
        rec = {
            "metric": "SS1 layer with fp8 (E4M3) input and weights on fp8 MFMA: dense-equiv TFLOP/s + % of "
                      "fp8 MFMA/HBM roofline",
            "value": wk["dense_flops"] / t / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": t * 1e3, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "fp8 e4m3 (x and W_c, per-row scales), fp32 accumulate, bf16 y",
            "data": "synthetic (seeded N(0,1) inputs, N(0,0.02) compressed weights, both quantized per row, "
                    "seeded balanced plan)",
            "config": {"workload": name + "_fp8a", "M": wl.M, "K": wl.K, "N": wl.N, "c": wl.c, "BK": wl.BK,
                       "BN": wl.BN, "kernel": "quantize_fp8 + fold8",
                       "cache": f"cold ({nsets} rotating buffer sets)", "forward_only_ms": t_fwd * 1e3,
                       "executed_fp8_tflops": wk["dense_flops"] / t_fwd / 1e12,
                       "bf16_layer_ms": t16 * 1e3, "speedup_vs_bf16_layer": t16 / t},
            "roofline": roof,
        }
        if args.no_cpu_baseline:
            rec["cpu_baseline"] = None
        else:
            rec["cpu_baseline"] = cpu_baseline_dtype(wl, np.float64, 8.0)
            rec["cpu_baseline"]["sample"] += " (the dequantized layer's arithmetic is the same)"
        print(json.dumps(rec), flush=True)
        return

    if args.op == "project":
        name = args.workload or PROJECT_HEADLINE
        rec, wl = measure_project(name, args.steps, args.warmup)
        rec["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_project(wl)
        print(json.dumps(rec), flush=True)
        return

    rec, wl = measure(args.workload or HEADLINE, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl, budget_s=8.0)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
