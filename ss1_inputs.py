"""Seeded synthetic inputs for the SS1 forward: the workloads' shapes, seeds and
value distributions, and nothing of the method's arithmetic.

This is the one module that both the tests/bench (driving the HIP library) and
the CPU oracle's callers share: it only draws numbers (NumPy PCG64) and encodes
float32 values as bf16 bit patterns (round to nearest, ties to even).  The plan
(hash and signs) is NOT drawn here: each side derives it from the plan seed
with its own SplitMix64.

Workloads (the shapes stand in for the models the SS1 summary page measures:
GPT-2 Small/Large MLP projections and Llama-3-8B projections; synthetic values
stand in for trained weights and activations):

* ``tiny``        M=64, K=256, N=256, c=2, BK=32, BN=32, float32; x ~ N(0,1),
                  W_c ~ U(-1/16, 1/16).
* ``gpt2s_up``    M=8192, K=768, N=3072, c=2, BK=64, BN=64, bf16.
* ``gpt2l_up``    M=8192, K=1280, N=5120, c=4, BK=64, BN=64, bf16.
* ``gpt2l_down``  M=8192, K=5120, N=1280, c=4, BK=64, BN=64, bf16.
* ``llama_gateup_m{1,16,4096}``  K=4096, N=14336, c=2, BK=64, BN=64, bf16.
* ``llama_down_m{1,16,4096}``    K=14336, N=4096, c=2, BK=64, BN=64, bf16.
* ``square_c{1,2,4,8}_bn{32,64,128}``  M=K=N=4096, BK=64, bf16.

bf16 workloads: x ~ N(0,1), W_c ~ N(0, 0.02) (standard deviation 0.02).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    cfg: int          # index of the workload family (0..4)
    layer: int        # sub-layer number inside the family
    M: int
    K: int
    N: int
    c: int
    BK: int
    BN: int
    dtype: str        # "f32" or "bf16"
    m_idx: int = 0    # which M of a family with several M values
    x_dist: str = "normal"
    w_dist: str = "normal002"

    @property
    def J(self):
        return self.K // self.BK

    @property
    def Jc(self):
        return self.J // self.c

    @property
    def Kc(self):
        return self.K // self.c

    @property
    def G(self):
        return self.N // self.BN

    @property
    def plan_seed(self):
        return 0x55310000 + 256 * self.cfg + self.layer

    @property
    def x_seed(self):
        return 0x55320000 + 256 * self.cfg + 16 * self.layer + self.m_idx

    @property
    def w_seed(self):
        return 0x55330000 + 256 * self.cfg + self.layer

    def with_m(self, M: int) -> "Workload":
        d = dict(self.__dict__)
        d["M"] = M
        return Workload(**d)


def _build_workloads():
    w = [Workload("tiny", 0, 0, 64, 256, 256, 2, 32, 32, "f32", 0, "normal", "uniform16"),
         Workload("gpt2s_up", 1, 0, 8192, 768, 3072, 2, 64, 64, "bf16"),
         Workload("gpt2l_up", 2, 0, 8192, 1280, 5120, 4, 64, 64, "bf16"),
         Workload("gpt2l_down", 2, 1, 8192, 5120, 1280, 4, 64, 64, "bf16")]
    for mi, M in enumerate((1, 16, 4096)):
        w.append(Workload(f"llama_gateup_m{M}", 3, 0, M, 4096, 14336, 2, 64, 64, "bf16", mi))
        w.append(Workload(f"llama_down_m{M}", 3, 1, M, 14336, 4096, 2, 64, 64, "bf16", mi))
    layer = 0
    for c in (1, 2, 4, 8):
        for BN in (32, 64, 128):
            w.append(Workload(f"square_c{c}_bn{BN}", 4, layer, 4096, 4096, 4096, c, 64, BN, "bf16"))
            layer += 1
    return {x.name: x for x in w}


WORKLOADS = _build_workloads()


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(a) -> np.ndarray:
    """Encode float32 values as bf16 bit patterns (uint16), rounding to nearest
    with ties to even.  Finite inputs only."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Decode bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw(dist: str, seed: int, shape) -> np.ndarray:
    """float32 values of one named distribution."""
    g = rng(seed)
    if dist == "normal":
        return g.standard_normal(shape, dtype=np.float32)
    if dist == "normal002":
        return (g.standard_normal(shape, dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    if dist == "uniform16":
        return g.uniform(-1.0 / 16, 1.0 / 16, size=shape).astype(np.float32)
    if dist == "int4":
        # integers in {-4..4}: every sum and product the layer forms stays an
        # exactly representable integer, so results can be compared bit for bit
        return g.integers(-4, 5, size=shape).astype(np.float32)
    raise ValueError(dist)


@dataclass
class Tensors:
    """Host copies of one workload's inputs.  For bf16 workloads ``x_bits`` and
    ``w_bits`` hold the uint16 patterns and ``x``/``w`` their exact float32
    values; for float32 workloads the bits fields are None."""
    x: np.ndarray
    w: np.ndarray
    x_bits: np.ndarray | None = None
    w_bits: np.ndarray | None = None
    meta: dict = field(default_factory=dict)


def make_inputs(wl: Workload, M: int | None = None, integer: bool = False,
                x_seed: int | None = None, w_seed: int | None = None) -> Tensors:
    """Inputs of workload ``wl`` (optionally with another M, integer-valued
    values, or other seeds)."""
    M = wl.M if M is None else M
    xs = wl.x_seed if x_seed is None else x_seed
    ws = wl.w_seed if w_seed is None else w_seed
    xd = "int4" if integer else wl.x_dist
    wd = "int4" if integer else wl.w_dist
    x = draw(xd, xs, (M, wl.K))
    w = draw(wd, ws, (wl.N, wl.Kc))
    if wl.dtype == "bf16":
        xb = f32_to_bf16_bits(x)
        wb = f32_to_bf16_bits(w)
        return Tensors(bf16_bits_to_f32(xb), bf16_bits_to_f32(wb), xb, wb)
    return Tensors(x, w)


def dense_weight_seed(wl: Workload) -> int:
    """Seed of the dense [N][K] weight that a projection test or benchmark
    projects onto the layer's sharing pattern."""
    return 0x55340000 + 256 * wl.cfg + wl.layer


def make_dense_weight(wl: Workload, integer: bool = False):
    """A dense [N][K] weight for projection: N(0, 0.02) (the GPT-2 init scale),
    or integers in {-4..4}.  Returns (float32 values, uint16 bf16 bits or
    None); for bf16 layers the values are the exact bf16 values."""
    w = draw("int4" if integer else "normal002", dense_weight_seed(wl), (wl.N, wl.K))
    if wl.dtype == "bf16":
        b = f32_to_bf16_bits(w)
        return bf16_bits_to_f32(b), b
    return w, None
