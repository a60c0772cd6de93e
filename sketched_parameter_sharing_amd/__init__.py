"""SS1 (Sketch Structured Transform) linear-layer forward for AMD MI355X.

The compute runs in ``libss1.so`` (hand-written HIP kernels for gfx950, C ABI
in ``include/ss1.h``); this package only marshals torch tensors and NumPy
arrays into that ABI.  Importing it does not load the library; the first call
does, and fails loudly when the library has not been built.
"""
from dataclasses import dataclass

from ._lib import (  # noqa: F401
    ALGOS,
    BF16,
    F32,
    EXPORTS,
    SS1Error,
    backward,
    backward_select_algo,
    forward,
    forward_fp8,
    forward_fp8w,
    forward_idx,
    forward_ws,
    forward_ws_query,
    load,
    mlp_forward,
    mlp_forward_static,
    plan,
    plan_index,
    project,
    quantize_fp8,
    select_algo,
    static_rows,
    sketch,
    version,
)


@dataclass
class DevicePlan:
    """A layer's plan made by the library on the host and copied to the GPU
    once: the forward hash/sign [G][J] and the inverse index idx/isign
    [G][Jc][c]."""
    K: int
    N: int
    c: int
    BK: int
    BN: int
    hash: object
    sign: object
    idx: object
    isign: object

    @classmethod
    def make(cls, seed: int, K: int, N: int, c: int, BK: int, BN: int, device="cuda"):
        import torch
        h, s = plan(seed, K, N, c, BK, BN)
        i, si = plan_index(h, s, K, N, c, BK, BN)
        t = lambda a: torch.from_numpy(a).to(device)
        return cls(K, N, c, BK, BN, t(h), t(s), t(i), t(si))

    def forward(self, x, W_c, y=None, algo="auto", use_index=False, stream=None):
        if use_index:
            return forward_idx(x, W_c, self.idx, self.isign, self.c, self.BK, self.BN, y, algo, stream)
        return forward(x, W_c, self.hash, self.sign, self.c, self.BK, self.BN, y, algo, stream)
