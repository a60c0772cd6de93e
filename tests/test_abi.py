"""Host-side tests of the C ABI (no GPU): the library loads and exports every
function ``include/ss1.h`` declares, the C++ plan equals the oracle's plan bit
for bit, and every argument check returns its status before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import sketched_parameter_sharing_amd as ss1
from sketched_parameter_sharing_amd import _lib
from ss1_inputs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "ss1.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ss1_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = _lib.load()
    declared = _declared_functions()
    assert declared, "no declarations parsed"
    assert sorted(declared) == sorted(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    assert ss1.version().count(".") == 2


def test_status_strings():
    lib = _lib.load()
    for code in range(8):
        assert lib.ss1_status_string(code).decode() not in ("", "unknown status")
    assert lib.ss1_status_string(99).decode() == "unknown status"


PLAN_CASES = sorted({(w.plan_seed, w.K, w.N, w.c, w.BK, w.BN) for w in WORKLOADS.values()}) + [
    (0, 48, 12, 3, 4, 3), (2**64 - 1, 64, 8, 8, 1, 8), (123, 4096, 32, 1, 1, 32),
    (77, 8 * 4096, 1, 4096, 8, 1),
]


@pytest.mark.parametrize("seed,K,N,c,BK,BN", PLAN_CASES)
def test_plan_matches_oracle_bit_exact(seed, K, N, c, BK, BN):
    if c > 64:
        pytest.skip("beyond the library's c limit")
    h, s = ss1.plan(seed, K, N, c, BK, BN)
    ho, so = oracle.plan(seed, K, N, c, BK, BN)
    assert h.dtype == np.int32 and s.dtype == np.int8
    assert np.array_equal(h, ho) and np.array_equal(s, so)
    idx, isg = ss1.plan_index(h, s, K, N, c, BK, BN)
    io, iso = oracle.plan_index(ho, so, K, N, c, BK, BN)
    assert np.array_equal(idx, io) and np.array_equal(isg, iso)


def test_plan_rejects_bad_chunking():
    for args in [(256, 256, 2, 30, 32), (256, 256, 3, 32, 32), (256, 250, 2, 32, 32),
                 (256, 256, 0, 32, 32), (-256, 256, 2, 32, 32), (256, 256, 65, 1, 32)]:
        with pytest.raises(ss1.SS1Error) as e:
            ss1.plan(1, *args)
        assert e.value.status == _lib.ERR_SHAPE
    with pytest.raises(ss1.SS1Error) as e:  # J = K/BK above the chunk limit
        ss1.plan(1, 8192, 4, 2, 1, 4)
    assert e.value.status == _lib.ERR_SHAPE
    lib = _lib.load()
    assert lib.ss1_plan(1, 64, 8, 2, 8, 4, None, None) == _lib.ERR_NULL


def test_plan_index_rejects_bad_plans():
    K, N, c, BK, BN = 64, 8, 2, 8, 4
    h, s = ss1.plan(3, K, N, c, BK, BN)
    for mutate in (lambda h, s: h.__setitem__((0, 0), 4),        # out of range
                   lambda h, s: h.__setitem__((0, 0), -1),
                   lambda h, s: s.__setitem__((1, 2), 0),        # not +-1
                   lambda h, s: s.__setitem__((1, 2), 2),
                   lambda h, s: h.__setitem__((1, 0), (h[1, 0] + 1) % 4)):  # unbalanced
        hh, sh = h.copy(), s.copy()
        mutate(hh, sh)
        with pytest.raises(ss1.SS1Error) as e:
            ss1.plan_index(hh, sh, K, N, c, BK, BN)
        assert e.value.status == _lib.ERR_PLAN
    lib = _lib.load()
    buf = np.zeros(64, dtype=np.int32)
    assert lib.ss1_plan_index(None, buf.ctypes.data, K, N, c, BK, BN, buf.ctypes.data,
                              buf.ctypes.data) == _lib.ERR_NULL


# ----------------------------------------------- forward / sketch arg checks
# Fake device addresses: every case below fails a host check, so the library
# returns before touching them or calling HIP.
A = 0x10000  # 16-byte aligned


def T(rows, cols, dtype=_lib.BF16, data=A, reserved=0):
    return _lib.Tensor(data, dtype, reserved, rows, cols)


def fwd(x, w, y, c=2, BK=64, BN=64, h=A, s=A, algo=None, idx=False):
    lib = _lib.load()
    args = [ctypes.byref(x), ctypes.byref(w), h, s, c, BK, BN, ctypes.byref(y)]
    if algo is None:
        f = lib.ss1_forward_idx if idx else lib.ss1_forward
        return f(*args, None)
    f = lib.ss1_forward_idx_algo if idx else lib.ss1_forward_algo
    return f(*args, algo, None)


FORWARD_ERRORS = [
    # (description, x, W_c, y, kwargs, expected)
    ("K % BK", T(8, 770), T(64, 385), T(8, 64), {}, _lib.ERR_SHAPE),
    ("J % c", T(8, 192), T(64, 64), T(8, 64), {"c": 2}, _lib.ERR_SHAPE),
    ("N % BN", T(8, 256), T(96, 128), T(8, 96), {}, _lib.ERR_SHAPE),
    ("W_c cols", T(8, 256), T(64, 256), T(8, 64), {}, _lib.ERR_SHAPE),
    ("y rows", T(8, 256), T(64, 128), T(9, 64), {}, _lib.ERR_SHAPE),
    ("y cols", T(8, 256), T(64, 128), T(8, 128), {}, _lib.ERR_SHAPE),
    ("negative M", T(-1, 256), T(64, 128), T(-1, 64), {}, _lib.ERR_SHAPE),
    ("bf16 BK % 8", T(8, 256), T(64, 128), T(8, 64), {"BK": 4}, _lib.ERR_SHAPE),
    ("f32 BK % 4", T(8, 256, _lib.F32), T(64, 128, _lib.F32), T(8, 64, _lib.F32), {"BK": 2}, _lib.ERR_SHAPE),
    ("c = 0", T(8, 256), T(64, 128), T(8, 64), {"c": 0}, _lib.ERR_SHAPE),
    ("c > max", T(8, 65 * 64), T(64, 64), T(8, 64), {"c": 65}, _lib.ERR_SHAPE),
    ("reserved", T(8, 256, reserved=1), T(64, 128), T(8, 64), {}, _lib.ERR_SHAPE),
    ("dtype mix", T(8, 256, _lib.F32), T(64, 128), T(8, 64), {}, _lib.ERR_DTYPE),
    ("y dtype", T(8, 256), T(64, 128), T(8, 64, _lib.F32), {}, _lib.ERR_DTYPE),
    ("bad dtype", T(8, 256, 7), T(64, 128, 7), T(8, 64, 7), {}, _lib.ERR_DTYPE),
    ("null x data", T(8, 256, data=None), T(64, 128), T(8, 64), {}, _lib.ERR_NULL),
    ("null y data", T(8, 256), T(64, 128), T(8, 64, data=None), {}, _lib.ERR_NULL),
    ("null W data", T(8, 256), T(64, 128, data=None), T(8, 64), {}, _lib.ERR_NULL),
    ("null hash", T(8, 256), T(64, 128), T(8, 64), {"h": None}, _lib.ERR_NULL),
    ("null sign", T(8, 256), T(64, 128), T(8, 64), {"s": None}, _lib.ERR_NULL),
    ("x align", T(8, 256, data=A + 2), T(64, 128), T(8, 64), {}, _lib.ERR_ALIGN),
    ("W align", T(8, 256), T(64, 128, data=A + 8), T(8, 64), {}, _lib.ERR_ALIGN),
    ("y align", T(8, 256), T(64, 128), T(8, 64, data=A + 4), {}, _lib.ERR_ALIGN),
    ("hash align", T(8, 256), T(64, 128), T(8, 64), {"h": A + 2}, _lib.ERR_ALIGN),
    ("algo fused f32", T(8, 256, _lib.F32), T(64, 128, _lib.F32), T(8, 64, _lib.F32),
     {"algo": _lib.ALGO_FUSED}, _lib.ERR_ALGO),
    ("algo fused BK", T(8, 256), T(64, 128), T(8, 64), {"BK": 16, "algo": _lib.ALGO_FUSED}, _lib.ERR_ALGO),
    ("algo fused BN", T(8, 256), T(48, 128), T(8, 48), {"BN": 48, "algo": _lib.ALGO_FUSED}, _lib.ERR_ALGO),
    ("algo smallm M", T(17, 256), T(64, 128), T(17, 64), {"algo": _lib.ALGO_SMALLM}, _lib.ERR_ALGO),
    ("algo smallm BN", T(4, 256), T(40, 128), T(4, 40), {"BN": 40, "algo": _lib.ALGO_SMALLM}, _lib.ERR_ALGO),
    ("algo gemv M", T(5, 2048), T(64, 1024), T(5, 64), {"algo": _lib.ALGO_GEMV}, _lib.ERR_ALGO),
    ("algo gemv Kc", T(1, 512), T(64, 256), T(1, 64), {"algo": _lib.ALGO_GEMV}, _lib.ERR_ALGO),
    ("algo gemv f32", T(1, 2048, _lib.F32), T(64, 1024, _lib.F32), T(1, 64, _lib.F32),
     {"algo": _lib.ALGO_GEMV}, _lib.ERR_ALGO),
    ("algo fold f32", T(8, 256, _lib.F32), T(64, 128, _lib.F32), T(8, 64, _lib.F32),
     {"algo": _lib.ALGO_FOLD}, _lib.ERR_ALGO),
    ("algo fold BK", T(8, 256), T(64, 128), T(8, 64), {"BK": 32, "algo": _lib.ALGO_FOLD}, _lib.ERR_ALGO),
    ("algo group f32", T(8, 256, _lib.F32), T(64, 128, _lib.F32), T(8, 64, _lib.F32),
     {"algo": _lib.ALGO_GROUP}, _lib.ERR_ALGO),
    ("algo group BK", T(8, 256), T(64, 128), T(8, 64), {"BK": 32, "algo": _lib.ALGO_GROUP}, _lib.ERR_ALGO),
    ("algo group c", T(8, 256), T(64, 256), T(8, 64), {"c": 1, "algo": _lib.ALGO_GROUP}, _lib.ERR_ALGO),
    ("algo group BN", T(8, 256), T(32, 128), T(8, 32), {"BN": 32, "algo": _lib.ALGO_GROUP}, _lib.ERR_ALGO),
    ("algo unknown", T(8, 256), T(64, 128), T(8, 64), {"algo": 10}, _lib.ERR_ALGO),
]


@pytest.mark.parametrize("idx", [False, True])
@pytest.mark.parametrize("desc,x,w,y,kw,expected", FORWARD_ERRORS, ids=[e[0] for e in FORWARD_ERRORS])
def test_forward_argument_checks(desc, x, w, y, kw, expected, idx):
    assert fwd(x, w, y, idx=idx, **kw) == expected


def test_forward_null_descriptors():
    lib = _lib.load()
    x, w, y = T(8, 256), T(64, 128), T(8, 64)
    assert lib.ss1_forward(None, ctypes.byref(w), A, A, 2, 64, 64, ctypes.byref(y), None) == _lib.ERR_NULL
    assert lib.ss1_forward(ctypes.byref(x), None, A, A, 2, 64, 64, ctypes.byref(y), None) == _lib.ERR_NULL
    assert lib.ss1_forward(ctypes.byref(x), ctypes.byref(w), A, A, 2, 64, 64, None, None) == _lib.ERR_NULL


def test_forward_m0_is_a_noop_without_hip():
    # M = 0 returns before any HIP call, even with null x / y data
    for algo in (None, _lib.ALGO_AUTO, _lib.ALGO_FUSED, _lib.ALGO_SMALLM, _lib.ALGO_GENERIC):
        assert fwd(T(0, 256, data=None), T(64, 128), T(0, 64, data=None), algo=algo) == _lib.OK


def _sk(x, z, c=2, BK=64, BN=64, N=128, h=A, s=A):
    return _lib.load().ss1_sketch(ctypes.byref(x), h, s, c, BK, BN, N, ctypes.byref(z), None)


def test_sketch_argument_checks():
    assert _sk(T(8, 256), T(15, 128)) == _lib.ERR_SHAPE            # z rows != G*M
    assert _sk(T(8, 256), T(16, 64)) == _lib.ERR_SHAPE             # z cols != K/c
    assert _sk(T(8, 250), T(16, 125)) == _lib.ERR_SHAPE            # K % BK
    assert _sk(T(8, 256, _lib.F32), T(16, 128, _lib.BF16)) == _lib.ERR_DTYPE
    assert _sk(T(8, 256, 5), T(16, 128)) == _lib.ERR_DTYPE
    assert _sk(T(8, 256), T(16, 128), h=None) == _lib.ERR_NULL
    assert _sk(T(8, 256, data=A + 2), T(16, 128)) == _lib.ERR_ALIGN
    assert _sk(T(8, 256), T(16, 128), h=A + 1) == _lib.ERR_ALIGN
    assert _sk(T(0, 256, data=None), T(0, 128, data=None)) == _lib.OK
    lib = _lib.load()
    assert lib.ss1_sketch(None, A, A, 2, 64, 64, 128, None, None) == _lib.ERR_NULL


def _pj(W, Wc, h=A, s=A, c=2, BK=64, BN=64):
    lib = _lib.load()
    return lib.ss1_project(ctypes.byref(W), h, s, c, BK, BN, ctypes.byref(Wc), None)


def test_project_argument_checks():
    assert _pj(T(128, 256), T(127, 128)) == _lib.ERR_SHAPE           # W_c rows != N
    assert _pj(T(128, 256), T(128, 64)) == _lib.ERR_SHAPE            # W_c cols != K/c
    assert _pj(T(128, 250), T(128, 125)) == _lib.ERR_SHAPE           # K % BK
    assert _pj(T(100, 256), T(100, 128)) == _lib.ERR_SHAPE           # N % BN
    assert _pj(T(128, 256), T(128, 128), c=3) == _lib.ERR_SHAPE      # J % c
    assert _pj(T(128, 256), T(128, 128), BK=4, c=2) == _lib.ERR_SHAPE  # bf16 needs BK % 8
    assert _pj(T(128, 256, _lib.F32), T(128, 128, _lib.BF16)) == _lib.ERR_DTYPE
    assert _pj(T(128, 256, 7), T(128, 128, 7)) == _lib.ERR_DTYPE
    assert _pj(T(128, 256, reserved=1), T(128, 128)) == _lib.ERR_SHAPE
    assert _pj(T(128, 256), T(128, 128), h=None) == _lib.ERR_NULL
    assert _pj(T(128, 256), T(128, 128), s=None) == _lib.ERR_NULL
    assert _pj(T(128, 256, data=None), T(128, 128)) == _lib.ERR_NULL
    assert _pj(T(128, 256, data=A + 2), T(128, 128)) == _lib.ERR_ALIGN
    assert _pj(T(128, 256), T(128, 128, data=A + 8)) == _lib.ERR_ALIGN
    assert _pj(T(128, 256), T(128, 128), h=A + 2) == _lib.ERR_ALIGN
    assert _pj(T(65536 * 64, 128), T(65536 * 64, 64)) == _lib.ERR_SHAPE  # G above 65535
    lib = _lib.load()
    assert lib.ss1_project(None, A, A, 2, 64, 64, ctypes.byref(T(128, 128)), None) == _lib.ERR_NULL
    assert lib.ss1_project(ctypes.byref(T(128, 256)), A, A, 2, 64, 64, None, None) == _lib.ERR_NULL


def _layer(rows, cols, c=2, BK=64, BN=64, h=A, s=A, dtype=_lib.BF16, reserved=0):
    return _lib.Layer(T(rows, cols, dtype), h, s, c, BK, BN, reserved)


def _mlp(x, up, down, h, y):
    lib = _lib.load()
    return lib.ss1_mlp_forward(ctypes.byref(x), ctypes.byref(up), ctypes.byref(down), ctypes.byref(h),
                               ctypes.byref(y), None)


def test_mlp_forward_argument_checks():
    up, down = _layer(512, 128), _layer(256, 256)          # 256 -> 512 -> 256, c = 2
    x, h, y = T(64, 256), T(32, 512), T(64, 256)
    assert _mlp(T(64, 250), up, down, h, y) == _lib.ERR_SHAPE        # x cols vs up K
    assert _mlp(x, _layer(512, 100), down, h, y) == _lib.ERR_SHAPE   # up W_c cols != K/c
    assert _mlp(x, up, _layer(256, 128), h, y) == _lib.ERR_SHAPE     # down K != up N
    assert _mlp(x, up, down, T(32, 500), y) == _lib.ERR_SHAPE        # h cols != up N
    assert _mlp(x, up, down, h, T(63, 256)) == _lib.ERR_SHAPE        # y rows != M
    assert _mlp(x, up, down, h, T(64, 255)) == _lib.ERR_SHAPE        # y cols != down N
    assert _mlp(x, up, down, T(0, 512), y) == _lib.ERR_SHAPE         # no workspace rows
    assert _mlp(x, _layer(512, 128, reserved=1), down, h, y) == _lib.ERR_SHAPE
    assert _mlp(x, up, down, T(32, 512, _lib.F32), y) == _lib.ERR_DTYPE
    assert _mlp(x, _layer(512, 128, dtype=_lib.F32), down, h, y) == _lib.ERR_DTYPE
    assert _mlp(x, _layer(512, 128, h=None), down, h, y) == _lib.ERR_NULL
    assert _mlp(x, up, _layer(256, 256, s=None), h, y) == _lib.ERR_NULL
    assert _mlp(T(64, 256, data=None), up, down, h, y) == _lib.ERR_NULL
    assert _mlp(x, up, down, T(32, 512, data=A + 2), y) == _lib.ERR_ALIGN
    assert _mlp(x, up, down, h, T(64, 256, data=A + 4)) == _lib.ERR_ALIGN
    assert _mlp(T(0, 256, data=None), up, down, T(0, 512, data=None), T(0, 256, data=None)) == _lib.OK
    lib = _lib.load()
    assert lib.ss1_mlp_forward(None, ctypes.byref(up), ctypes.byref(down), ctypes.byref(h),
                               ctypes.byref(y), None) == _lib.ERR_NULL


def test_quantize_fp8_argument_checks():
    lib = _lib.load()
    F8 = _lib.FP8_E4M3

    def q(W, Q, sc=A):
        return lib.ss1_quantize_fp8(ctypes.byref(W), ctypes.byref(Q), sc, None)

    assert q(T(64, 128), T(64, 127, F8)) == _lib.ERR_SHAPE
    assert q(T(64, 127), T(64, 127, F8)) == _lib.ERR_SHAPE          # odd Kc
    assert q(T(64, 128), T(64, 128)) == _lib.ERR_DTYPE              # Q not FP8
    assert q(T(64, 128, F8), T(64, 128, F8)) == _lib.ERR_DTYPE      # W_c not BF16/F32
    assert q(T(64, 128), T(64, 128, F8), sc=None) == _lib.ERR_NULL
    assert q(T(64, 128), T(64, 128, F8), sc=A + 2) == _lib.ERR_ALIGN
    assert q(T(64, 128, data=A + 8), T(64, 128, F8)) == _lib.ERR_ALIGN
    assert q(T(0, 128, data=None), T(0, 128, F8, data=None), sc=None) == _lib.OK
    assert lib.ss1_quantize_fp8(None, ctypes.byref(T(1, 2, F8)), A, None) == _lib.ERR_NULL


def test_forward_fp8w_argument_checks():
    lib = _lib.load()
    F8 = _lib.FP8_E4M3

    def f(x, Q, y, sc=A, c=2, BK=64, BN=64):
        return lib.ss1_forward_fp8w(ctypes.byref(x), ctypes.byref(Q), sc, A, A, c, BK, BN, ctypes.byref(y), None)

    assert f(T(300, 256), T(64, 128), T(300, 64)) == _lib.ERR_DTYPE          # Q not FP8
    assert f(T(300, 256, _lib.F32), T(64, 128, F8), T(300, 64, _lib.F32)) == _lib.ERR_DTYPE
    assert f(T(300, 256), T(64, 100, F8), T(300, 64)) == _lib.ERR_SHAPE      # Q cols != K/c
    assert f(T(300, 240), T(48, 120, F8), T(300, 48), BK=24, BN=48) == _lib.ERR_SHAPE  # no fp8 kernel
    assert f(T(300, 256), T(96, 128, F8), T(300, 96), BN=48) == _lib.ERR_SHAPE  # BN 48 needs M <= 16
    assert f(T(300, 256), T(64, 128, F8), T(300, 64), sc=None) == _lib.ERR_NULL
    assert f(T(300, 256), T(64, 128, F8), T(300, 64), sc=A + 1) == _lib.ERR_ALIGN
    assert f(T(0, 256, data=None), T(64, 128, F8), T(0, 64, data=None)) == _lib.OK


def test_backward_argument_checks():
    lib = _lib.load()

    def b(x, w, dy, dx, dw, c=2, BK=64, BN=64, h=A, s=A):
        return lib.ss1_backward(ctypes.byref(x), ctypes.byref(w), h, s, c, BK, BN, ctypes.byref(dy),
                                ctypes.byref(dx) if dx is not None else None,
                                ctypes.byref(dw) if dw is not None else None, None)

    x, w, dy, dx, dw = T(96, 512), T(128, 256), T(96, 128), T(96, 512), T(128, 256)
    assert b(x, w, dy, None, None) == _lib.OK                                   # nothing asked
    assert b(T(96, 512, _lib.F32), T(128, 256, _lib.F32), T(96, 128, _lib.F32), dx, dw) == _lib.ERR_DTYPE
    assert b(T(96, 480), T(128, 240), dy, T(96, 480), T(128, 240), BK=48) == _lib.ERR_SHAPE  # BK % 32
    assert b(x, T(96, 256), T(96, 96), dx, T(96, 256), BN=48) == _lib.ERR_SHAPE            # BN % 32
    assert b(x, w, T(95, 128), dx, dw) == _lib.ERR_SHAPE                         # dy rows
    assert b(x, w, dy, T(96, 511), dw) == _lib.ERR_SHAPE                         # dx cols
    assert b(x, w, dy, dx, T(128, 255)) == _lib.ERR_SHAPE                        # dW_c cols
    assert b(x, w, dy, T(96, 512, _lib.F32), dw) == _lib.ERR_DTYPE
    assert b(x, w, dy, dx, T(128, 256, data=None)) == _lib.ERR_NULL
    assert b(x, w, dy, dx, dw, h=None) == _lib.ERR_NULL
    assert b(x, w, dy, T(96, 512, data=A + 2), dw) == _lib.ERR_ALIGN
    assert b(x, w, dy, dx, T(128, 256, data=A + 4)) == _lib.ERR_ALIGN
    assert lib.ss1_backward(None, ctypes.byref(w), A, A, 2, 64, 64, ctypes.byref(dy), None, None,
                            None) == _lib.ERR_NULL


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(4, 256, dtype=torch.bfloat16)
    w = torch.zeros(64, 128, dtype=torch.bfloat16)
    h = torch.zeros(1, 4, dtype=torch.int32)
    with pytest.raises(ValueError):
        ss1.forward(x, w, h, h.to(torch.int8), 2, 64, 64)


def test_select_algo_host():
    # decode shapes take the matrix-vector kernel (M <= 4) or the small-M
    # kernel, float32 the generic one; invalid shapes give the forward's own
    # status codes
    assert ss1.select_algo(1, 4096, 14336, 2, 64, 64) == "gemv"
    assert ss1.select_algo(2, 14336, 4096, 2, 64, 64) == "gemv"
    assert ss1.select_algo(4, 4096, 14336, 2, 64, 64) == "gemv"
    assert ss1.select_algo(4, 14336, 4096, 2, 64, 64) == "smallm"  # 896-thread blocks at 4 token slots
    assert ss1.select_algo(3, 65536, 1024, 2, 64, 64) == "smallm"  # Kc = 32768 > 16384 at 4 token slots
    # the decode kernel needs 128 KB of LDS for K = 4096 (the host sees the
    # device's LDS size; without a device it assumes 64 KB)
    assert ss1.select_algo(5, 4096, 14336, 2, 64, 64) in ("decode", "smallm")
    assert ss1.select_algo(16, 14336, 4096, 2, 64, 64) == "smallm"
    assert ss1.select_algo(1, 768, 3072, 2, 64, 64) == "smallm"   # Kc = 384: under one wave of slices
    assert ss1.select_algo(64, 256, 256, 2, 32, 32, "f32") == "generic"
    assert ss1.select_algo(300, 240, 96, 2, 24, 48) == "generic"
    assert ss1.select_algo(4096, 4096, 4096, 2, 64, 64) in ("fused", "band", "fold")
    # E4M3 weights: the choice of ss1_forward_fp8w (no band or generic kernel)
    assert ss1.select_algo(1, 4096, 14336, 2, 64, 64, weights="fp8") == "gemv"
    assert ss1.select_algo(8, 4096, 14336, 2, 64, 64, weights="fp8") == "smallm"  # decode: bf16 weights only
    assert ss1.select_algo(8192, 768, 3072, 2, 64, 64, weights="fp8") in ("fused", "fold")
    with pytest.raises(ss1.SS1Error) as e:
        ss1.select_algo(64, 256, 256, 2, 32, 32, "f32", weights="fp8")
    assert e.value.status == _lib.ERR_DTYPE
    with pytest.raises(ss1.SS1Error) as e:   # neither small-M nor fused: BN = 48
        ss1.select_algo(300, 768, 3 * 48, 2, 32, 48, weights="fp8")
    assert e.value.status == _lib.ERR_SHAPE
    with pytest.raises(ss1.SS1Error) as e:
        ss1.select_algo(8, 250, 64, 2, 64, 64)
    assert e.value.status == _lib.ERR_SHAPE
    lib = _lib.load()
    out = ctypes.c_int32(0)
    assert lib.ss1_select_algo(None, ctypes.byref(T(1, 1)), 2, 64, 64, ctypes.byref(out)) == _lib.ERR_NULL
    assert lib.ss1_select_algo(ctypes.byref(T(8, 256)), ctypes.byref(T(64, 128)), 2, 64, 64, None) == _lib.ERR_NULL


def test_backward_select_algo_host():
    # the kernels ss1_backward reports; its checks are ss1_backward's own
    dx_k, dw_k = ss1.backward_select_algo(300, 768, 192, 2, 64, 64)
    assert dx_k in ("fold", "generic") and dw_k in ("fold", "fused")
    with pytest.raises(ss1.SS1Error) as e:
        ss1.backward_select_algo(96, 480, 128, 2, 48, 64)       # BK % 32
    assert e.value.status == _lib.ERR_SHAPE
    lib = _lib.load()
    a, b = ctypes.c_int32(0), ctypes.c_int32(0)
    assert lib.ss1_backward_select_algo(None, ctypes.byref(T(1, 1)), 2, 64, 64, ctypes.byref(a),
                                        ctypes.byref(b)) == _lib.ERR_NULL
    assert lib.ss1_backward_select_algo(ctypes.byref(T(8, 256, _lib.F32)), ctypes.byref(T(64, 128, _lib.F32)), 2,
                                        64, 64, ctypes.byref(a), ctypes.byref(b)) == _lib.ERR_DTYPE


def test_binding_checks_plan_and_scale_arrays():
    # the ABI reads plan arrays and row scales by pointer alone, so the binding
    # checks their element type, layout and size before any call
    torch = pytest.importorskip("torch")
    K, N, c, BK, BN = 512, 128, 2, 64, 64          # G = 2, J = 8, Jc = 4
    h = torch.zeros(2, 8, dtype=torch.int32)
    s = torch.ones(2, 8, dtype=torch.int8)
    _lib._check_plan(h, s, K, N, c, BK, BN)         # well formed
    with pytest.raises(ValueError, match="hash must be torch.int32"):
        _lib._check_plan(h.to(torch.int64), s, K, N, c, BK, BN)
    with pytest.raises(ValueError, match="sign must be torch.int8"):
        _lib._check_plan(h, s.to(torch.int32), K, N, c, BK, BN)
    with pytest.raises(ValueError, match="hold 16 elements"):
        _lib._check_plan(h[:, :7].contiguous(), s, K, N, c, BK, BN)
    with pytest.raises(ValueError, match="contiguous"):
        _lib._check_plan(torch.zeros(8, 4, dtype=torch.int32).T, s, K, N, c, BK, BN)
    idx = torch.zeros(2, 4, 2, dtype=torch.int32)
    _lib._check_plan(idx, s.view(2, 4, 2), K, N, c, BK, BN, index=True)
    with pytest.raises(ValueError, match="idx must hold 16"):
        _lib._check_plan(idx[:1], s.view(2, 4, 2), K, N, c, BK, BN, index=True)
    sc = torch.ones(N, dtype=torch.float32)
    _lib._check_vec(sc, torch.float32, N, "scale")
    with pytest.raises(ValueError, match="scale must be torch.float32"):
        _lib._check_vec(sc.double(), torch.float32, N, "scale")
    with pytest.raises(ValueError, match="scale must hold 128"):
        _lib._check_vec(sc[:-1], torch.float32, N, "scale")


def test_mlp_forward_static_argument_checks():
    # checks that run before any HIP call: a row of h wider than the static
    # array, a null descriptor, a dtype the library has no kernel for
    lib = _lib.load()
    N1 = (_lib.STATIC_SCRATCH_BYTES // 2) + 64          # one bf16 row of h > the array
    up = _lib.Layer(T(N1, 128), A, A, 2, 64, 64, 0)
    down = _lib.Layer(T(64, N1 // 2), A, A, 2, 64, 64, 0)
    x, y = T(8, 256), T(8, 64)
    f = lib.ss1_mlp_forward_static
    assert f(ctypes.byref(x), ctypes.byref(up), ctypes.byref(down), ctypes.byref(y), None) == _lib.ERR_SHAPE
    assert f(None, ctypes.byref(up), ctypes.byref(down), ctypes.byref(y), None) == _lib.ERR_NULL
    assert f(ctypes.byref(T(8, 256, 7)), ctypes.byref(up), ctypes.byref(down), ctypes.byref(y),
             None) == _lib.ERR_DTYPE
    # M == 0 only checks the descriptors (no device needed)
    up = _lib.Layer(T(3072, 384), A, A, 2, 64, 64, 0)
    down = _lib.Layer(T(768, 1536), A, A, 2, 64, 64, 0)
    assert f(ctypes.byref(T(0, 768, data=None)), ctypes.byref(up), ctypes.byref(down),
             ctypes.byref(T(0, 768, data=None)), None) == _lib.OK
    assert f(ctypes.byref(T(0, 768, data=None)), ctypes.byref(up), ctypes.byref(down),
             ctypes.byref(T(0, 700, data=None)), None) == _lib.ERR_SHAPE
    assert _lib.static_rows(5120, 2) == 3072 and _lib.static_rows(N1 - 64, 2) == 1


def test_binding_constants_match_the_header():
    # the binding's kernel, status and dtype codes are the header's enum values
    text = open(os.path.join(ROOT, "include", "ss1.h")).read()
    enum = {m.group(1): int(m.group(2)) for m in re.finditer(r"\b(SS1_[A-Z0-9_]+)\s*=\s*(-?\d+)", text)}
    for name, code in _lib.ALGOS.items():
        assert enum[f"SS1_ALGO_{name.upper()}"] == code, name
    assert enum["SS1_OK"] == _lib.OK and enum["SS1_ERR_ALGO"] == _lib.ERR_ALGO
    assert (enum["SS1_F32"], enum["SS1_BF16"], enum["SS1_FP8_E4M3"]) == (_lib.F32, _lib.BF16, _lib.FP8_E4M3)
