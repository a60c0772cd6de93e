"""Build libss1.so (the SS1 forward library) in-tree with hipcc for gfx950.

Run as ``python -m sketched_parameter_sharing_amd.build`` or call ``build()``.
Host sources (.cpp) and device sources (.hip) compile to objects in
``_build/`` next to this file and link into ``libss1.so`` beside it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libss1.so")
BUILD_DIR = os.path.join(HERE, "_build")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # keep the compiler from forming packed float32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Per-source options.  The fold kernels keep 128 float32 accumulators per
# lane; with MFMA results in ordinary VGPRs they fit beside the operands, while
# the compiler's default (accumulators in AGPRs, other values spilled there)
# copies about a hundred registers back and forth on every k-stage.
EXTRA = {
    "ss1_fold.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "ss1_group.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libss1.so)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".cpp", ".hip")))


def _stale(src: str, obj: str) -> bool:
    """An object is stale when it is missing or older than its source or any
    header beside the sources (every source includes some of them)."""
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    deps = [src] + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    return any(os.path.getmtime(d) > t for d in deps)


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compile every source (only stale objects with ``incremental``) and
    link libss1.so; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        if incremental and not _stale(src, obj):
            return obj
        cmd = [hipcc, *COMMON, *EXTRA.get(os.path.basename(src), []), f"--offload-arch={ARCH}", "-c", src,
               "-o", obj]
        if src.endswith(".cpp"):
            cmd = [hipcc, *COMMON, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = (r.stdout + r.stderr).strip()
        # the host pass does not know the packed-fp32 feature name and says so
        lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n" + "\n".join(lines))
        if verbose and lines:
            print("\n".join(lines), file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = OUT + ".tmp"
    # every symbol resolved at link time: a missing definition fails the build
    # instead of the first load
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, OUT)
    build_peaks()
    return OUT


PEAKS_SRC = os.path.join(HERE, "peaks", "ss1_peaks.hip")
PEAKS_OUT = os.path.join(HERE, "libss1_peaks.so")


def build_peaks() -> str:
    """The benchmark's machine-rate probes (MFMA, L2, LDS-DMA, HBM, LDS) as
    their own library; the SS1 library does not link them."""
    tmp = PEAKS_OUT + ".tmp"
    cmd = [_hipcc(), *COMMON, "-Wno-inline-asm", "-mllvm", "-amdgpu-mfma-vgpr-form=1", f"--offload-arch={ARCH}",
           "-shared", PEAKS_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, PEAKS_OUT)
    return PEAKS_OUT


if __name__ == "__main__":
    print(build(verbose=True, incremental="--incremental" in sys.argv))
