"""ctypes binding of libss1.so: argument marshalling only.

Every step of the SS1 forward runs in the library's HIP kernels; this module
turns torch tensors (device memory) and NumPy arrays (host plan arrays) into
the pointers and sizes of the C ABI declared in ``include/ss1.h``.  It raises
:class:`SS1Error` for any non-zero status and refuses to run at all when the
library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; SS1_LIBRARY may name another build of the same ABI
LIB_PATH = os.environ.get("SS1_LIBRARY") or os.path.join(HERE, "libss1.so")

# status codes (ss1_status)
OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_PLAN, ERR_ALIGN, ERR_HIP, ERR_ALGO = range(8)
# dtypes (ss1_dtype)
F32, BF16, FP8_E4M3 = 0, 1, 2
# kernel choice (ss1_algo)
(ALGO_AUTO, ALGO_FUSED, ALGO_SMALLM, ALGO_GENERIC, ALGO_BAND, ALGO_FOLD, ALGO_GEMV, ALGO_DECODE, ALGO_SPLIT,
 ALGO_GROUP) = range(10)
ALGOS = {"auto": ALGO_AUTO, "fused": ALGO_FUSED, "smallm": ALGO_SMALLM, "generic": ALGO_GENERIC,
         "band": ALGO_BAND, "fold": ALGO_FOLD, "gemv": ALGO_GEMV, "decode": ALGO_DECODE, "split": ALGO_SPLIT,
         "group": ALGO_GROUP}

EXPORTS = ("ss1_version", "ss1_status_string", "ss1_plan", "ss1_plan_index", "ss1_forward",
           "ss1_forward_idx", "ss1_forward_algo", "ss1_forward_idx_algo", "ss1_select_algo", "ss1_sketch",
           "ss1_project", "ss1_mlp_forward", "ss1_quantize_fp8", "ss1_forward_fp8w",
           "ss1_backward", "ss1_backward_select_algo", "ss1_mlp_forward_static", "ss1_forward_fp8",
           "ss1_forward_ws_query", "ss1_forward_ws")
ALGO_NAMES = {v: k for k, v in ALGOS.items()}


class SS1Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _status_string(status) if _LIB is not None else str(status)
        super().__init__(f"{where}: status {status} ({msg})")


class Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class Layer(ctypes.Structure):
    _fields_ = [("W_c", Tensor), ("hash", ctypes.c_void_p), ("sign", ctypes.c_void_p),
                ("c", ctypes.c_int32), ("BK", ctypes.c_int32), ("BN", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


_LIB = None


def load():
    """Load libss1.so (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m sketched_parameter_sharing_amd.build` (needs hipcc)")
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, u64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p
    tp = ctypes.POINTER(Tensor)
    lib.ss1_version.restype = ctypes.c_char_p
    lib.ss1_version.argtypes = []
    lib.ss1_status_string.restype = ctypes.c_char_p
    lib.ss1_status_string.argtypes = [i32]
    lib.ss1_plan.restype = i32
    lib.ss1_plan.argtypes = [u64, i64, i64, i32, i32, i32, vp, vp]
    lib.ss1_plan_index.restype = i32
    lib.ss1_plan_index.argtypes = [vp, vp, i64, i64, i32, i32, i32, vp, vp]
    for name in ("ss1_forward", "ss1_forward_idx"):
        f = getattr(lib, name)
        f.restype = i32
        f.argtypes = [tp, tp, vp, vp, i32, i32, i32, tp, vp]
    for name in ("ss1_forward_algo", "ss1_forward_idx_algo"):
        f = getattr(lib, name)
        f.restype = i32
        f.argtypes = [tp, tp, vp, vp, i32, i32, i32, tp, i32, vp]
    lib.ss1_sketch.restype = i32
    lib.ss1_sketch.argtypes = [tp, vp, vp, i32, i32, i32, i64, tp, vp]
    lib.ss1_project.restype = i32
    lib.ss1_project.argtypes = [tp, vp, vp, i32, i32, i32, tp, vp]
    lib.ss1_mlp_forward.restype = i32
    lib.ss1_mlp_forward.argtypes = [tp, ctypes.POINTER(Layer), ctypes.POINTER(Layer), tp, tp, vp]
    lib.ss1_mlp_forward_static.restype = i32
    lib.ss1_mlp_forward_static.argtypes = [tp, ctypes.POINTER(Layer), ctypes.POINTER(Layer), tp, vp]
    lib.ss1_quantize_fp8.restype = i32
    lib.ss1_quantize_fp8.argtypes = [tp, tp, vp, vp]
    lib.ss1_forward_fp8.restype = i32
    lib.ss1_forward_fp8.argtypes = [tp, vp, tp, vp, vp, vp, i32, i32, i32, tp, vp]
    lib.ss1_forward_fp8w.restype = i32
    lib.ss1_forward_fp8w.argtypes = [tp, tp, vp, vp, vp, i32, i32, i32, tp, vp]
    lib.ss1_backward.restype = i32
    lib.ss1_backward.argtypes = [tp, tp, vp, vp, i32, i32, i32, tp, tp, tp, vp]
    lib.ss1_forward_ws_query.restype = i32
    lib.ss1_forward_ws_query.argtypes = [tp, tp, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(i32)]
    lib.ss1_forward_ws.restype = i32
    lib.ss1_forward_ws.argtypes = [tp, tp, vp, vp, i32, i32, i32, tp, vp, ctypes.c_size_t, vp]
    lib.ss1_select_algo.restype = i32
    lib.ss1_select_algo.argtypes = [tp, tp, i32, i32, i32, ctypes.POINTER(i32)]
    lib.ss1_backward_select_algo.restype = i32
    lib.ss1_backward_select_algo.argtypes = [tp, tp, i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    _LIB = lib
    return lib


def _status_string(s: int) -> str:
    return load().ss1_status_string(int(s)).decode()


def _check(status: int, where: str):
    if status != OK:
        raise SS1Error(status, where)


def version() -> str:
    return load().ss1_version().decode()


# ------------------------------------------------------------------ host plan
def _np_ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def plan(seed: int, K: int, N: int, c: int, BK: int, BN: int):
    """Seeded balanced plan from the library (host): int32 hash [G][J], int8
    sign [G][J]."""
    if K <= 0 or BK <= 0 or N <= 0 or BN <= 0 or K % BK or N % BN:
        _check(load().ss1_plan(seed, K, N, c, BK, BN, None, None), "ss1_plan")
    G, J = N // BN, K // BK
    h = np.empty((G, J), dtype=np.int32)
    s = np.empty((G, J), dtype=np.int8)
    _check(load().ss1_plan(int(seed) & (2**64 - 1), K, N, c, BK, BN, _np_ptr(h), _np_ptr(s)), "ss1_plan")
    return h, s


def plan_index(hash_, sign, K: int, N: int, c: int, BK: int, BN: int):
    """Validated inverse index from the library (host): int32 idx [G][Jc][c]
    and int8 isign [G][Jc][c]."""
    h = np.ascontiguousarray(hash_, dtype=np.int32)
    s = np.ascontiguousarray(sign, dtype=np.int8)
    G, J = N // BN, K // BK
    if h.size != G * J or s.size != G * J:
        raise ValueError("plan arrays do not match (K, N, BK, BN)")
    idx = np.empty(h.size, dtype=np.int32)
    isg = np.empty(h.size, dtype=np.int8)
    _check(load().ss1_plan_index(_np_ptr(h), _np_ptr(s), K, N, c, BK, BN, _np_ptr(idx), _np_ptr(isg)),
           "ss1_plan_index")
    Jc = J // c
    return idx.reshape(G, Jc, c), isg.reshape(G, Jc, c)


# ------------------------------------------------------------- device calls
def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    if t.dtype in (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8)):
        return FP8_E4M3  # OCP E4M3 codes (quantized weights only)
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16, float32, or uint8 / float8_e4m3fn codes)")


def _desc(t) -> Tensor:
    if t.dim() != 2 or not t.is_contiguous():
        raise ValueError("matrices must be 2-D and contiguous")
    return Tensor(t.data_ptr() if t.numel() else None, _dtype_code(t), 0, t.shape[0], t.shape[1])


def _stream(stream) -> int | None:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream or None


def _check_device(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("device entry points take GPU tensors")


def _check_vec(t, dtype, numel: int, what: str):
    """A device array the C ABI reads by pointer alone (a plan array, a row
    scale): it must have the element type the kernels read, be contiguous and
    hold exactly ``numel`` elements, since the library cannot see its size."""
    if t.dtype != dtype:
        raise ValueError(f"{what} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{what} must hold {numel} elements, got {t.numel()}")


def _plan_sizes(K: int, N: int, c: int, BK: int, BN: int):
    """(G*J, G*Jc*c) for a layer, or None when the chunking does not divide
    (the library then reports the shape error itself)."""
    if min(K, N, c, BK, BN) <= 0 or K % BK or N % BN or (K // BK) % c:
        return None
    G, J = N // BN, K // BK
    return G * J, G * (J // c) * c


def _check_plan(hash_, sign, K: int, N: int, c: int, BK: int, BN: int, index: bool = False):
    import torch
    n = _plan_sizes(K, N, c, BK, BN)
    if n is None:
        return
    numel = n[1] if index else n[0]
    names = ("idx", "isign") if index else ("hash", "sign")
    _check_vec(hash_, torch.int32, numel, names[0])
    _check_vec(sign, torch.int8, numel, names[1])


def forward(x, W_c, hash_, sign, c: int, BK: int, BN: int, y=None, algo: str = "auto", stream=None):
    """y = SS1(x) on the GPU (ss1_forward / ss1_forward_algo).  ``hash_`` and
    ``sign`` are device tensors (int32 / int8) of shape [G][J]."""
    import torch
    _check_device(x, W_c, hash_, sign)
    _check_plan(hash_, sign, x.shape[-1], W_c.shape[0], c, BK, BN)
    if y is None:
        y = torch.empty((x.shape[0], W_c.shape[0]), dtype=x.dtype, device=x.device)
    dx, dw, dy = _desc(x), _desc(W_c), _desc(y)
    lib = load()
    if algo == "auto":
        st = lib.ss1_forward(ctypes.byref(dx), ctypes.byref(dw), hash_.data_ptr(), sign.data_ptr(),
                             c, BK, BN, ctypes.byref(dy), _stream(stream))
    else:
        st = lib.ss1_forward_algo(ctypes.byref(dx), ctypes.byref(dw), hash_.data_ptr(), sign.data_ptr(),
                                  c, BK, BN, ctypes.byref(dy), ALGOS[algo], _stream(stream))
    _check(st, "ss1_forward")
    return y


def forward_ws_query(M: int, K: int, N: int, c: int, BK: int, BN: int, dtype: int = BF16):
    """(kernel name, workspace bytes) of ss1_forward_ws for a layer of these
    sizes (ss1_forward_ws_query; no data is read)."""
    dx = Tensor(None, dtype, 0, M, K)
    dw = Tensor(None, dtype, 0, N, K // c if c > 0 else 0)
    nbytes, algo = ctypes.c_size_t(0), ctypes.c_int32(0)
    _check(load().ss1_forward_ws_query(ctypes.byref(dx), ctypes.byref(dw), c, BK, BN, ctypes.byref(nbytes),
                                       ctypes.byref(algo)), "ss1_forward_ws_query")
    return ALGO_NAMES[algo.value], nbytes.value


def forward_ws(x, W_c, hash_, sign, c: int, BK: int, BN: int, workspace=None, y=None, stream=None):
    """y = SS1(x) on the GPU with a caller-owned workspace (ss1_forward_ws).
    ``workspace`` is a device tensor of at least the bytes forward_ws_query
    reports (allocated here when None and needed)."""
    import torch
    _check_device(x, W_c, hash_, sign)
    _check_plan(hash_, sign, x.shape[-1], W_c.shape[0], c, BK, BN)
    if y is None:
        y = torch.empty((x.shape[0], W_c.shape[0]), dtype=x.dtype, device=x.device)
    dx, dw, dy = _desc(x), _desc(W_c), _desc(y)
    lib = load()
    if workspace is None:
        nbytes, algo = ctypes.c_size_t(0), ctypes.c_int32(0)
        _check(lib.ss1_forward_ws_query(ctypes.byref(dx), ctypes.byref(dw), c, BK, BN, ctypes.byref(nbytes),
                                        ctypes.byref(algo)), "ss1_forward_ws_query")
        if nbytes.value:
            workspace = torch.empty(nbytes.value, dtype=torch.uint8, device=x.device)
    wp, wb = (workspace.data_ptr(), workspace.numel() * workspace.element_size()) if workspace is not None else (None, 0)
    st = lib.ss1_forward_ws(ctypes.byref(dx), ctypes.byref(dw), hash_.data_ptr(), sign.data_ptr(), c, BK, BN,
                            ctypes.byref(dy), wp, wb, _stream(stream))
    _check(st, "ss1_forward_ws")
    return y


def forward_idx(x, W_c, idx, isign, c: int, BK: int, BN: int, y=None, algo: str = "auto", stream=None):
    """As :func:`forward` with the inverse index (device int32 / int8
    tensors [G][Jc][c]) instead of the forward hash."""
    import torch
    _check_device(x, W_c, idx, isign)
    _check_plan(idx, isign, x.shape[-1], W_c.shape[0], c, BK, BN, index=True)
    if y is None:
        y = torch.empty((x.shape[0], W_c.shape[0]), dtype=x.dtype, device=x.device)
    dx, dw, dy = _desc(x), _desc(W_c), _desc(y)
    lib = load()
    if algo == "auto":
        st = lib.ss1_forward_idx(ctypes.byref(dx), ctypes.byref(dw), idx.data_ptr(), isign.data_ptr(),
                                 c, BK, BN, ctypes.byref(dy), _stream(stream))
    else:
        st = lib.ss1_forward_idx_algo(ctypes.byref(dx), ctypes.byref(dw), idx.data_ptr(), isign.data_ptr(),
                                      c, BK, BN, ctypes.byref(dy), ALGOS[algo], _stream(stream))
    _check(st, "ss1_forward_idx")
    return y


def mlp_forward(x, up, down, h=None, y=None, row_chunk: int | None = None, stream=None):
    """SS1 MLP pair on the GPU (ss1_mlp_forward): y = SS1_down(GELU(SS1_up(x))).
    ``up`` and ``down`` are (W_c, hash, sign, c, BK, BN) tuples of device
    tensors and ints.  ``h`` is the [R][N1] workspace (allocated with
    R = row_chunk, default all rows, when None); returns (h, y)."""
    import torch
    Wu, hu, su, cu, BKu, BNu = up
    Wd, hd, sd, cd, BKd, BNd = down
    _check_device(x, Wu, hu, su, Wd, hd, sd)
    _check_plan(hu, su, x.shape[-1], Wu.shape[0], cu, BKu, BNu)
    _check_plan(hd, sd, Wu.shape[0], Wd.shape[0], cd, BKd, BNd)
    M = x.shape[0]
    if h is None:
        R = max(1, min(M, row_chunk or M))
        h = torch.empty((R, Wu.shape[0]), dtype=x.dtype, device=x.device)
    if y is None:
        y = torch.empty((M, Wd.shape[0]), dtype=x.dtype, device=x.device)
    lu = Layer(_desc(Wu), hu.data_ptr(), su.data_ptr(), cu, BKu, BNu, 0)
    ld = Layer(_desc(Wd), hd.data_ptr(), sd.data_ptr(), cd, BKd, BNd, 0)
    dx, dh, dy = _desc(x), _desc(h), _desc(y)
    st = load().ss1_mlp_forward(ctypes.byref(dx), ctypes.byref(lu), ctypes.byref(ld), ctypes.byref(dh),
                                ctypes.byref(dy), _stream(stream))
    _check(st, "ss1_mlp_forward")
    return h, y


# Bytes of the library's static h workspace (SS1_STATIC_SCRATCH_BYTES).
STATIC_SCRATCH_BYTES = 32 << 20


def static_rows(N1: int, dtype_bytes: int) -> int:
    """Rows per chunk ss1_mlp_forward_static uses for an up-projection of N1
    neurons (the header's formula)."""
    R = STATIC_SCRATCH_BYTES // (N1 * dtype_bytes)
    return R - R % 256 if R >= 256 else R


def mlp_forward_static(x, up, down, y=None, stream=None):
    """SS1 MLP pair on the GPU with no workspace argument and no allocation in
    the library (ss1_mlp_forward_static): h lives in the library's static
    device array.  Allocates y only when it is None; returns y."""
    import torch
    Wu, hu, su, cu, BKu, BNu = up
    Wd, hd, sd, cd, BKd, BNd = down
    _check_device(x, Wu, hu, su, Wd, hd, sd)
    _check_plan(hu, su, x.shape[-1], Wu.shape[0], cu, BKu, BNu)
    _check_plan(hd, sd, Wu.shape[0], Wd.shape[0], cd, BKd, BNd)
    if y is None:
        y = torch.empty((x.shape[0], Wd.shape[0]), dtype=x.dtype, device=x.device)
    lu = Layer(_desc(Wu), hu.data_ptr(), su.data_ptr(), cu, BKu, BNu, 0)
    ld = Layer(_desc(Wd), hd.data_ptr(), sd.data_ptr(), cd, BKd, BNd, 0)
    dx, dy = _desc(x), _desc(y)
    st = load().ss1_mlp_forward_static(ctypes.byref(dx), ctypes.byref(lu), ctypes.byref(ld), ctypes.byref(dy),
                                       _stream(stream))
    _check(st, "ss1_mlp_forward_static")
    return y


def quantize_fp8(W_c, Q=None, scale=None, stream=None):
    """Per-row E4M3 quantization on the GPU (ss1_quantize_fp8): returns
    (Q as uint8 codes [N][Kc], scale float32 [N])."""
    import torch
    _check_device(W_c)
    if Q is None:
        Q = torch.empty(W_c.shape, dtype=torch.uint8, device=W_c.device)
    if scale is None:
        scale = torch.empty((W_c.shape[0],), dtype=torch.float32, device=W_c.device)
    _check_device(Q, scale)
    _check_vec(scale, torch.float32, W_c.shape[0], "scale")
    dw, dq = _desc(W_c), _desc(Q)
    st = load().ss1_quantize_fp8(ctypes.byref(dw), ctypes.byref(dq), scale.data_ptr(), _stream(stream))
    _check(st, "ss1_quantize_fp8")
    return Q, scale


def forward_fp8w(x, Q, scale, hash_, sign, c: int, BK: int, BN: int, y=None, stream=None):
    """y = SS1(x) with fp8 compressed weights on the GPU (ss1_forward_fp8w)."""
    import torch
    _check_device(x, Q, scale, hash_, sign)
    _check_plan(hash_, sign, x.shape[-1], Q.shape[0], c, BK, BN)
    _check_vec(scale, torch.float32, Q.shape[0], "scale")
    if y is None:
        y = torch.empty((x.shape[0], Q.shape[0]), dtype=x.dtype, device=x.device)
    dx, dq, dy = _desc(x), _desc(Q), _desc(y)
    st = load().ss1_forward_fp8w(ctypes.byref(dx), ctypes.byref(dq), scale.data_ptr(), hash_.data_ptr(),
                                 sign.data_ptr(), c, BK, BN, ctypes.byref(dy), _stream(stream))
    _check(st, "ss1_forward_fp8w")
    return y


def forward_fp8(xq, xscale, Q, wscale, hash_, sign, c: int, BK: int, BN: int, y=None, stream=None):
    """y = SS1 with fp8 (E4M3) input and weights on the fp8 matrix cores
    (ss1_forward_fp8): ``xq``/``xscale`` from quantize_fp8(x), ``Q``/``wscale``
    from quantize_fp8(W_c); y is bf16."""
    import torch
    _check_device(xq, xscale, Q, wscale, hash_, sign)
    _check_plan(hash_, sign, xq.shape[-1], Q.shape[0], c, BK, BN)
    _check_vec(xscale, torch.float32, xq.shape[0], "xscale")
    _check_vec(wscale, torch.float32, Q.shape[0], "wscale")
    if y is None:
        y = torch.empty((xq.shape[0], Q.shape[0]), dtype=torch.bfloat16, device=xq.device)
    dx, dq, dy = _desc(xq), _desc(Q), _desc(y)
    st = load().ss1_forward_fp8(ctypes.byref(dx), xscale.data_ptr(), ctypes.byref(dq), wscale.data_ptr(),
                                hash_.data_ptr(), sign.data_ptr(), c, BK, BN, ctypes.byref(dy), _stream(stream))
    _check(st, "ss1_forward_fp8")
    return y


def backward(x, W_c, hash_, sign, c: int, BK: int, BN: int, dy, dx=True, dW_c=True, stream=None):
    """Gradients of the SS1 forward on the GPU (ss1_backward): returns
    (dx, dW_c); pass dx=None or dW_c=None to skip one, True to allocate it."""
    import torch
    _check_device(x, W_c, hash_, sign, dy)
    _check_plan(hash_, sign, x.shape[-1], W_c.shape[0], c, BK, BN)
    if dx is True:
        dx = torch.empty_like(x)
    if dW_c is True:
        dW_c = torch.empty_like(W_c)
    ddx = _desc(dx) if dx is not None else None
    ddw = _desc(dW_c) if dW_c is not None else None
    st = load().ss1_backward(ctypes.byref(_desc(x)), ctypes.byref(_desc(W_c)), hash_.data_ptr(), sign.data_ptr(),
                             c, BK, BN, ctypes.byref(_desc(dy)), ctypes.byref(ddx) if ddx else None,
                             ctypes.byref(ddw) if ddw else None, _stream(stream))
    _check(st, "ss1_backward")
    return dx, dW_c


def select_algo(M: int, K: int, N: int, c: int, BK: int, BN: int, dtype: str = "bf16",
                weights: str | None = None) -> str:
    """Name of the kernel ss1_forward runs for this layer ("fused", "smallm",
    "gemv", "band", "fold" or "generic"); with weights="fp8", the kernel
    ss1_forward_fp8w runs (bf16 x)."""
    code = BF16 if dtype == "bf16" else F32
    wcode = FP8_E4M3 if weights == "fp8" else code
    x = Tensor(None, code, 0, M, K)
    w = Tensor(None, wcode, 0, N, K // c if c > 0 else 0)
    out = ctypes.c_int32(-1)
    _check(load().ss1_select_algo(ctypes.byref(x), ctypes.byref(w), c, BK, BN, ctypes.byref(out)),
           "ss1_select_algo")
    return ALGO_NAMES[out.value]


def backward_select_algo(M: int, K: int, N: int, c: int, BK: int, BN: int):
    """Kernels ss1_backward runs for this layer (bf16): a pair of names
    (dx kernel, dW_c kernel).  "fold" forms no sketch; a dW_c kernel named
    "fused" contracts the sketch rounded to bf16; a dx kernel named "generic"
    is a tiled kernel that forms no sketch either."""
    x = Tensor(None, BF16, 0, M, K)
    w = Tensor(None, BF16, 0, N, K // c if c > 0 else 0)
    a, b = ctypes.c_int32(-1), ctypes.c_int32(-1)
    _check(load().ss1_backward_select_algo(ctypes.byref(x), ctypes.byref(w), c, BK, BN, ctypes.byref(a),
                                           ctypes.byref(b)), "ss1_backward_select_algo")
    return ALGO_NAMES[a.value], ALGO_NAMES[b.value]


def sketch(x, hash_, sign, c: int, BK: int, BN: int, N: int, z=None, out_dtype=None, stream=None):
    """Standalone sketch on the GPU (ss1_sketch): returns z as a [G*M][K/c]
    tensor (float32 by default, or ``out_dtype``)."""
    import torch
    _check_device(x, hash_, sign)
    _check_plan(hash_, sign, x.shape[-1], N, c, BK, BN)
    G = N // BN
    if z is None:
        z = torch.empty((G * x.shape[0], x.shape[1] // c), dtype=out_dtype or torch.float32, device=x.device)
    dx, dz = _desc(x), _desc(z)
    st = load().ss1_sketch(ctypes.byref(dx), hash_.data_ptr(), sign.data_ptr(), c, BK, BN, N,
                           ctypes.byref(dz), _stream(stream))
    _check(st, "ss1_sketch")
    return z


def project(W, hash_, sign, c: int, BK: int, BN: int, W_c=None, stream=None):
    """Least-squares projection of a dense [N][K] weight onto the SS1 sharing
    pattern on the GPU (ss1_project): returns W_c, [N][K/c], W's dtype."""
    import torch
    _check_device(W, hash_, sign)
    _check_plan(hash_, sign, W.shape[-1], W.shape[0], c, BK, BN)
    if W_c is None:
        W_c = torch.empty((W.shape[0], W.shape[1] // c), dtype=W.dtype, device=W.device)
    dw, dc = _desc(W), _desc(W_c)
    st = load().ss1_project(ctypes.byref(dw), hash_.data_ptr(), sign.data_ptr(), c, BK, BN,
                            ctypes.byref(dc), _stream(stream))
    _check(st, "ss1_project")
    return W_c
