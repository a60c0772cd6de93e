"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Plans: the library's ``ss1_plan`` output goes to the GPU, the oracle builds
its own plan from the same seed (the two are checked equal on the CPU).

Bars (written in each test):
* float32 layers: max|y - y_ref| / max|y_ref| <= 1e-5 (y_ref float64 oracle).
* bf16 layers: max|y - y_ref| / max|y_ref| <= 2e-2, and elementwise against
  the oracle's mirror (float32 sketch rounded to bf16, float64 contraction):
  |y - y_mirror| <= 2^-7 |y_mirror| + 1e-5 max|y_mirror| (one bf16 ulp plus
  float32 accumulation-order slack).  The fold kernel multiplies x by the
  expanded weight and never rounds a sketch, so its mirror is the float64
  oracle itself, under the same bound.
* integer-valued inputs: every intermediate is an exact integer, so float32
  output equals the oracle exactly and bf16 output equals the oracle rounded to
  bf16 (nearest, ties to even) bit for bit.
* standalone sketch: bit-exact against the oracle's float32 mirror sketch.
"""
import numpy as np
import pytest

import oracle
import sketched_parameter_sharing_amd as ss1
from ss1_inputs import WORKLOADS, Workload, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ss1.load()


# ------------------------------------------------------------------ helpers
def dev(t, wl_dtype):
    """Host inputs -> device tensor of the layer's dtype."""
    if wl_dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(t).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(t, dtype=np.float32)).cuda()


def host(y):
    """Device output -> float64 numpy (bf16 decoded exactly)."""
    if y.dtype == torch.bfloat16:
        return bf16_bits_to_f32(y.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return y.cpu().numpy().astype(np.float64)


def bits(y):
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


def device_plan(wl):
    return ss1.DevicePlan.make(wl.plan_seed, wl.K, wl.N, wl.c, wl.BK, wl.BN)


def oracle_plan(wl):
    return oracle.plan(wl.plan_seed, wl.K, wl.N, wl.c, wl.BK, wl.BN)


def run(wl, inp, plan, algo="auto", use_index=False, rows=None):
    xs = inp.x_bits if wl.dtype == "bf16" else inp.x
    ws = inp.w_bits if wl.dtype == "bf16" else inp.w
    x = dev(xs, wl.dtype)
    w = dev(ws, wl.dtype)
    y = plan.forward(x, w, algo=algo, use_index=use_index)
    torch.cuda.synchronize()
    return y


def rel_err(y, ref):
    scale = np.max(np.abs(ref)) if ref.size else 1.0
    return float(np.max(np.abs(y - ref)) / scale) if ref.size else 0.0


def kernel_of(wl, algo):
    """The kernel a call with this algo runs (auto resolved by the library)."""
    return ss1.select_algo(wl.M, wl.K, wl.N, wl.c, wl.BK, wl.BN, wl.dtype) if algo == "auto" else algo


def check_bf16(wl, inp, y, rows=None, kernel=None):
    """Tolerance gate against the float64 oracle plus the mirror check, on all
    rows or on the given sample of rows.  ``kernel`` is the kernel that ran
    (None: one of the sketch kernels)."""
    h, s = oracle_plan(wl)
    x = inp.x if rows is None else inp.x[rows]
    yg = host(y) if rows is None else host(y)[rows]
    ref = oracle.forward(x, inp.w, h, s, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    err = rel_err(yg, ref)
    assert err <= TOL_BF16, f"{wl.name}: normwise error {err:.3e} > {TOL_BF16}"
    if kernel == "fold":
        mir = ref
    else:
        mir = oracle.forward_mirror(x, inp.w, h, s, wl.K, wl.N, wl.c, wl.BK, wl.BN, sketch_bf16=True)
    top = np.max(np.abs(mir)) if mir.size else 0.0
    bad = np.abs(yg - mir) > 2.0 ** -7 * np.abs(mir) + 1e-5 * top
    assert not bad.any(), f"{wl.name}: {int(bad.sum())} outputs off the mirror oracle by more than one bf16 ulp"
    return err


# ------------------------------------------------------------ float32 path
def test_tiny_fp32_parity():
    wl = WORKLOADS["tiny"]
    inp = make_inputs(wl)
    y = run(wl, inp, device_plan(wl))
    h, s = oracle_plan(wl)
    ref = oracle.forward(inp.x, inp.w, h, s, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    yh = host(y)
    assert rel_err(yh, ref) <= TOL_F32
    big = np.abs(ref) >= 1e-2 * np.max(np.abs(ref))
    assert np.max(np.abs(yh - ref)[big] / np.abs(ref)[big]) <= 1e-4


def test_tiny_fp32_identity_plan_is_dense():
    # c = 1 with the identity plan must be the dense layer y = x W^T
    wl = WORKLOADS["tiny"]
    M, K, N, BK, BN = wl.M, wl.K, wl.N, wl.BK, wl.BN
    rng = np.random.Generator(np.random.PCG64(wl.x_seed))
    x = rng.standard_normal((M, K), dtype=np.float32)
    W = rng.uniform(-1 / 16, 1 / 16, size=(N, K)).astype(np.float32)
    G, J = N // BN, K // BK
    h = torch.arange(J, dtype=torch.int32).repeat(G, 1).contiguous().cuda()
    s = torch.ones((G, J), dtype=torch.int8).cuda()
    y = ss1.forward(dev(x, "f32"), dev(W, "f32"), h, s, 1, BK, BN)
    torch.cuda.synchronize()
    ref = x.astype(np.float64) @ W.astype(np.float64).T
    assert rel_err(host(y), ref) <= TOL_F32


def test_tiny_fp32_integer_exact():
    wl = WORKLOADS["tiny"]
    inp = make_inputs(wl, integer=True)
    y = run(wl, inp, device_plan(wl))
    h, s = oracle_plan(wl)
    ref = oracle.forward(inp.x, inp.w, h, s, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    assert np.array_equal(host(y), ref)


# --------------------------------------------------------------- bf16 path
BF16_NAMES = ["gpt2s_up", "gpt2l_up", "gpt2l_down", "llama_gateup_m4096", "llama_down_m4096"] + [
    f"square_c{c}_bn{bn}" for c in (1, 2, 4, 8) for bn in (32, 64, 128)]


@pytest.mark.parametrize("name", BF16_NAMES)
@pytest.mark.parametrize("algo", ["auto", "fused", "band", "generic", "fold", "group"])
def test_bf16_reduced_m(name, algo):
    # M = 300: two full 128-row tiles and a ragged tail (and a ragged band;
    # for the fold kernel one 256-row tile and a ragged one)
    wl = WORKLOADS[name].with_m(300)
    if algo == "generic" and wl.N * wl.K > 4096 * 4096:
        pytest.skip("generic kernel checked on the smaller layers")
    inp = make_inputs(wl)
    try:
        y = run(wl, inp, device_plan(wl), algo=algo)
    except ss1.SS1Error as e:
        assert e.status == 7 and algo in ("band", "group")
        pytest.skip("input rows too long for the band kernel" if algo == "band"
                    else "the group kernel takes c in {2, 4, 8}, BK % 64 == 0, BN of 64 or 128")
    err = check_bf16(wl, inp, y, kernel=kernel_of(wl, algo))
    print(f"{name} algo={algo} err={err:.3e}", flush=True)


@pytest.mark.parametrize("name", BF16_NAMES + ["llama_gateup_m16", "llama_down_m16",
                                               "llama_gateup_m1", "llama_down_m1"])
def test_bf16_full_size_sampled_rows(name):
    wl = WORKLOADS[name]
    inp = make_inputs(wl)
    y = run(wl, inp, device_plan(wl))
    rng = np.random.Generator(np.random.PCG64(99))
    if wl.M <= 64:
        rows = np.arange(wl.M)
    else:
        rows = np.unique(np.concatenate([[0, wl.M - 1], rng.choice(wl.M, 62, replace=False)]))
    assert np.isfinite(host(y)).all()
    err = check_bf16(wl, inp, y, rows, kernel=kernel_of(wl, "auto"))
    print(f"{name} full M={wl.M} kernel={kernel_of(wl, 'auto')} err={err:.3e}", flush=True)


@pytest.mark.parametrize("name,algo", [("gpt2s_up", "fused"), ("gpt2l_down", "fused"),
                                       ("llama_gateup_m16", "smallm"), ("llama_down_m16", "smallm"),
                                       ("llama_gateup_m16", "decode"),
                                       ("llama_gateup_m1", "gemv"), ("llama_down_m1", "gemv"),
                                       ("square_c8_bn128", "fused"), ("square_c1_bn32", "fused"),
                                       ("gpt2l_up", "generic"), ("gpt2s_up", "band"),
                                       ("gpt2l_up", "band"), ("gpt2s_up", "fold"),
                                       ("llama_down_m4096", "fold"), ("square_c1_bn128", "fold"),
                                       ("square_c8_bn32", "fold"), ("llama_gateup_m4096", "group"),
                                       ("gpt2l_down", "group"), ("square_c4_bn64", "group"),
                                       ("square_c8_bn128", "group")])
def test_bf16_integer_bit_exact(name, algo):
    wl = WORKLOADS[name]
    wl = wl.with_m(min(wl.M, {"smallm": 16, "decode": 16, "gemv": 4}.get(algo, 300)))
    inp = make_inputs(wl, integer=True)
    y = run(wl, inp, device_plan(wl), algo=algo)
    h, s = oracle_plan(wl)
    ref = oracle.forward(inp.x, inp.w, h, s, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    assert np.max(np.abs(ref)) < 2 ** 24
    expect = f32_to_bf16_bits(ref.astype(np.float32))
    assert np.array_equal(bits(y), expect)


@pytest.mark.parametrize("name", ["llama_gateup_m16", "llama_down_m16"])
@pytest.mark.parametrize("M", [1, 2, 5, 16])
def test_smallm_parity(name, M):
    wl = WORKLOADS[name].with_m(M)
    inp = make_inputs(wl)
    p = device_plan(wl)
    y = run(wl, inp, p, algo="smallm")
    check_bf16(wl, inp, y)
    if M > 4 and kernel_of(wl, "auto") == "smallm":
        ya = run(wl, inp, p)  # auto picks the same kernel
        assert torch.equal(y, ya)


@pytest.mark.parametrize("M", [1, 2, 5, 9, 16])
def test_decode_parity(M):
    # Llama-3-8B gate/up at decode sizes: 16 input rows of 4096 in LDS, one
    # group per block; rows past M read zeros and are not stored
    wl = WORKLOADS["llama_gateup_m16"].with_m(M)
    inp = make_inputs(wl)
    p = device_plan(wl)
    y = run(wl, inp, p, algo="decode")
    check_bf16(wl, inp, y, kernel="decode")
    assert torch.equal(y, run(wl, inp, p, algo="decode", use_index=True))
    if M > 4:
        assert kernel_of(wl, "auto") == "decode"
        assert torch.equal(y, run(wl, inp, p))


@pytest.mark.parametrize("M,K,N,c,BK,BN", [(16, 1024, 4096, 2, 32, 32), (11, 2048, 8192, 4, 64, 64),
                                           (7, 512, 1024, 1, 32, 64), (16, 3072, 2048, 3, 64, 64),
                                           (3, 1536, 768, 8, 32, 32), (5, 4096, 1024, 1, 64, 64)])
def test_decode_shapes(M, K, N, c, BK, BN):
    # both group widths, runtime c (3, 4, 8) and compile-time c (2), c = 1, Kc
    # that does not split evenly over the 8 waves (some waves get no k-step),
    # and 16 k-steps per wave (two batches of weight loads); against the
    # oracle and bit-exact on integer inputs
    wl = Workload("decode", 9, 6, M, K, N, c, BK, BN, "bf16")
    inp = make_inputs(wl)
    p = device_plan(wl)
    y = run(wl, inp, p, algo="decode")
    check_bf16(wl, inp, y, kernel="decode")
    inp = make_inputs(wl, integer=True)
    y = run(wl, inp, p, algo="decode")
    h, s = oracle_plan(wl)
    ref = oracle.forward(inp.x, inp.w, h, s, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    assert np.array_equal(bits(y), f32_to_bf16_bits(ref.astype(np.float32)))


@pytest.mark.parametrize("M,K,N,BN", [(7, 1024, 12288, 32), (16, 2048, 12288, 128), (3, 4096, 14336, 64)])
def test_smallm_column_block_pairs(M, K, N, BN):
    # layers with at least 384 pairs of 16-neuron blocks run two per small-M
    # block, sharing each wave's sketch (BN = 32: one pair per group; 128: two)
    wl = Workload("pairs", 9, 5, M, K, N, 2, 32, BN, "bf16")
    inp = make_inputs(wl)
    p = device_plan(wl)
    y = run(wl, inp, p, algo="smallm")
    check_bf16(wl, inp, y)
    assert torch.equal(y, run(wl, inp, p, algo="smallm", use_index=True))
    inp = make_inputs(wl, integer=True)
    y = run(wl, inp, p, algo="smallm")
    h, s = oracle_plan(wl)
    ref = oracle.forward(inp.x, inp.w, h, s, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    assert np.array_equal(bits(y), f32_to_bf16_bits(ref.astype(np.float32)))


@pytest.mark.parametrize("name,M", [("llama_gateup_m1", 1), ("llama_gateup_m1", 2), ("llama_gateup_m1", 3),
                                    ("llama_gateup_m1", 4), ("llama_down_m1", 1), ("llama_down_m1", 2)])
def test_gemv_parity(name, M):
    # one, two or four token slots (M = 3: a zero fourth token); 256 threads
    # per block for Llama gate/up, 896 for down (one 8-column slice each;
    # down takes the small-M kernel at four token slots)
    wl = WORKLOADS[name].with_m(M)
    inp = make_inputs(wl)
    p = device_plan(wl)
    y = run(wl, inp, p, algo="gemv")
    err = check_bf16(wl, inp, y, kernel="gemv")
    print(f"{name} M={M} gemv err={err:.3e}", flush=True)
    assert torch.equal(y, run(wl, inp, p))  # auto picks the same kernel at M <= 4
    assert torch.equal(y, run(wl, inp, p, algo="gemv", use_index=True))


@pytest.mark.parametrize("M,K,N,c,BK,BN", [
    (1, 1024, 128, 1, 64, 64),      # c = 1: the dense layer
    (3, 2400, 64, 2, 40, 32),       # 150 slices: 192 threads, BK = 40
    (2, 6144, 96, 3, 64, 48),       # c at run time, 48-neuron groups
    (4, 16384, 64, 4, 64, 16),      # four token slots, 512 threads (the limit for four)
    (1, 1024, 32, 2, 8, 16),        # 64 threads; J = 128, twice the block
    (1, 32768, 32, 2, 64, 16),      # two slices per thread
    (2, 65536, 32, 2, 64, 32),      # four slices per thread with two tokens
    (1, 131072, 16, 2, 64, 16),     # eight slices per thread, J = 2048 (twice the block)
])
def test_gemv_shapes(M, K, N, c, BK, BN):
    wl = Workload("gemv", 9, 4, M, K, N, c, BK, BN, "bf16")
    inp = make_inputs(wl)
    p = device_plan(wl)
    y = run(wl, inp, p, algo="gemv")
    check_bf16(wl, inp, y, kernel="gemv")
    assert torch.equal(y, run(wl, inp, p, algo="gemv", use_index=True))
    # integer-valued inputs: every partial sum is an exact integer
    inp = make_inputs(wl, integer=True)
    y = run(wl, inp, p, algo="gemv")
    h, s = oracle_plan(wl)
    ref = oracle.forward(inp.x, inp.w, h, s, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    assert np.max(np.abs(ref)) < 2 ** 24
    assert np.array_equal(bits(y), f32_to_bf16_bits(ref.astype(np.float32)))
    # every output is written
    yn = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    p.forward(dev(inp.x_bits, "bf16"), dev(inp.w_bits, "bf16"), y=yn, algo="gemv")
    torch.cuda.synchronize()
    assert torch.equal(yn, y)


@pytest.mark.parametrize("M,K,N,c,BK,BN", [
    (200, 384, 128, 3, 64, 64),     # runtime c on the fused kernel
    (130, 640, 256, 5, 64, 128),
    (77, 1920, 96, 3, 32, 32),
    (9, 2048, 64, 2, 32, 16),       # smallm with BN = 16
    (33, 240, 96, 2, 24, 48),       # generic: BK % 32 != 0, BN not 32/64/128
    (65, 160, 30, 5, 8, 3),
    (1, 64, 8, 8, 8, 8),
    (129, 512, 64, 1, 32, 64),
    (300, 1024, 256, 8, 32, 64),    # band: the sketch on the matrix cores, four source pairs
    (150, 512, 128, 4, 32, 32),     # band: two source pairs, BN = 32
    (100, 768, 256, 2, 32, 128),    # band: 32-wide steps, BN = 128
])
def test_bf16_odd_shapes(M, K, N, c, BK, BN):
    wl = Workload("odd", 9, 0, M, K, N, c, BK, BN, "bf16")
    inp = make_inputs(wl)
    p = device_plan(wl)
    ys = {}
    for algo in ("auto", "fused", "smallm", "gemv", "decode", "band", "generic", "fold"):
        try:
            ys[algo] = run(wl, inp, p, algo=algo)
        except ss1.SS1Error as e:
            assert e.status == 7  # kernel not applicable to this shape
            continue
        check_bf16(wl, inp, ys[algo], kernel=kernel_of(wl, algo))
    assert "auto" in ys and "generic" in ys


@pytest.mark.parametrize("name", ["llama_gateup_m4096", "square_c4_bn128", "square_c8_bn64", "gpt2l_down"])
def test_group_full_size_sampled_rows(name):
    # full size: blocks that run several token tiles through one pipeline
    # (the last one ragged where M is not a multiple of the tile)
    wl = WORKLOADS[name]
    if name == "gpt2l_down":
        wl = wl.with_m(wl.M - 77)
    inp = make_inputs(wl)
    y = run(wl, inp, device_plan(wl), algo="group")
    rng = np.random.Generator(np.random.PCG64(7))
    rows = np.unique(np.concatenate([[0, wl.M - 1], rng.choice(wl.M, 62, replace=False)]))
    assert np.isfinite(host(y)).all()
    err = check_bf16(wl, inp, y, rows, kernel="group")
    print(f"{name} group full M={wl.M} err={err:.3e}", flush=True)


@pytest.mark.parametrize("M,K,N,c,BK,BN", [(300, 1024, 256, 8, 32, 64), (150, 512, 128, 4, 32, 32),
                                           (77, 1280, 320, 4, 64, 64), (100, 768, 256, 2, 32, 128),
                                           (64, 768, 192, 2, 64, 64)])
def test_band_matrix_core_sketch_integer_bit_exact(M, K, N, c, BK, BN):
    # c = 2, 4, 8 on the band kernel form the sketch by MFMA against a signed
    # selection: with integer inputs every sum is exact, so y is the oracle
    # rounded to bf16 bit for bit
    wl = Workload("band_int", 11, 0, M, K, N, c, BK, BN, "bf16")
    inp = make_inputs(wl, integer=True)
    y = run(wl, inp, device_plan(wl), algo="band")
    h, s = oracle_plan(wl)
    ref = oracle.forward(inp.x, inp.w, h, s, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    assert np.max(np.abs(ref)) < 2 ** 24
    assert np.array_equal(bits(y), f32_to_bf16_bits(ref.astype(np.float32)))


@pytest.mark.parametrize("name,algo", [("gpt2s_up", "fused"), ("llama_down_m16", "smallm"),
                                       ("llama_gateup_m16", "decode"),
                                       ("gpt2l_up", "generic"), ("tiny", "generic"),
                                       ("gpt2s_up", "band"), ("gpt2l_up", "band"),
                                       ("gpt2s_up", "fold"), ("llama_gateup_m4096", "fold"),
                                       ("llama_gateup_m4096", "group"), ("square_c8_bn128", "group"),
                                       ("gpt2l_down", "group")])
def test_hash_and_index_forms_agree(name, algo):
    wl = WORKLOADS[name]
    wl = wl.with_m(min(wl.M, 256))
    inp = make_inputs(wl)
    p = device_plan(wl)
    y1 = run(wl, inp, p, algo=algo)
    y2 = run(wl, inp, p, algo=algo, use_index=True)
    y3 = run(wl, inp, p, algo=algo)
    assert torch.equal(y1, y2) and torch.equal(y1, y3)  # same bits, run to run


def test_m0_is_noop_and_y_fully_written():
    wl = WORKLOADS["gpt2s_up"]
    p = device_plan(wl)
    x = torch.empty((0, wl.K), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((wl.N, wl.Kc), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((0, wl.N), dtype=torch.bfloat16, device="cuda")
    ss1.forward(x, w, p.hash, p.sign, wl.c, wl.BK, wl.BN, y)
    for algo in ("fold", "band", "fused", "group"):
        ss1.forward(x, w, p.hash, p.sign, wl.c, wl.BK, wl.BN, y, algo=algo)
    # every output is written: start from NaN
    wl2 = wl.with_m(131)
    inp = make_inputs(wl2)
    for algo in ("fused", "band", "generic", "fold", "group"):
        y = torch.full((131, wl.N), float("nan"), dtype=torch.bfloat16, device="cuda")
        p.forward(dev(inp.x_bits, "bf16"), dev(inp.w_bits, "bf16"), y=y, algo=algo)
        torch.cuda.synchronize()
        assert torch.isfinite(y).all()


@pytest.mark.parametrize("name,M", [("gpt2s_up", 1), ("gpt2s_up", 77), ("gpt2s_up", 128), ("gpt2s_up", 129),
                                    ("gpt2l_down", 300), ("square_c2_bn128", 513), ("square_c2_bn128", 4000),
                                    ("llama_down_m4096", 40)])
def test_fold_tile_shapes(name, M):
    # 128 x 128 tiles (M <= 128); 192 x 256 tiles where one round of them holds
    # the layer, with a ragged last row tile; 256 x 256 tiles with a ragged
    # last row tile (M = 4000: 256 such tiles, one round, against 336 of 192
    # rows); 128-neuron groups (two per tile); and a 14336-long K
    wl = WORKLOADS[name].with_m(M)
    inp = make_inputs(wl)
    y = run(wl, inp, device_plan(wl), algo="fold")
    print(f"{name} M={M} fold err={check_bf16(wl, inp, y, kernel='fold'):.3e}", flush=True)


def test_fold_192_row_tiles_full_size():
    # GPT-2 L down (M = 8192, N = 1280): 160 tiles of 256 rows would leave 96
    # compute units idle, so the fold runs 43 x 5 tiles of 192 rows; the last
    # row tile holds 128 rows
    wl = WORKLOADS["gpt2l_down"]
    inp = make_inputs(wl)
    y = run(wl, inp, device_plan(wl), algo="fold")
    rng = np.random.Generator(np.random.PCG64(7))
    rows = np.unique(np.concatenate([[0, 191, 192, 8063, 8064, wl.M - 1], rng.choice(wl.M, 40, replace=False)]))
    assert np.isfinite(host(y)).all()
    err = check_bf16(wl, inp, y, rows, kernel="fold")
    print(f"gpt2l_down full M fold err={err:.3e}", flush=True)


def test_fold_split_launch():
    # 16 x 20 tiles of 256 x 256 end in a partial round: the first 4096
    # neurons run as 256 x 256 tiles, the last 1024 as 128 x 256 tiles
    wl = Workload("split", 9, 3, 4096, 256, 5120, 2, 64, 64, "bf16")
    inp = make_inputs(wl)
    y = run(wl, inp, device_plan(wl), algo="fold")
    check_bf16(wl, inp, y, kernel="fold")
    inp = make_inputs(wl, integer=True)
    y = run(wl, inp, device_plan(wl), algo="fold")
    h, s = oracle_plan(wl)
    ref = oracle.forward(inp.x, inp.w, h, s, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    assert np.array_equal(bits(y), f32_to_bf16_bits(ref.astype(np.float32)))


def test_fold_neuron_tile_of_128():
    # N = 384 is not a multiple of 256: 256 x 128 tiles of 4 waves
    wl = Workload("n384", 9, 1, 300, 512, 384, 2, 64, 64, "bf16")
    inp = make_inputs(wl)
    y = run(wl, inp, device_plan(wl), algo="fold")
    check_bf16(wl, inp, y, kernel="fold")
    inp = make_inputs(wl, integer=True)
    y = run(wl, inp, device_plan(wl), algo="fold")
    h, s = oracle_plan(wl)
    ref = oracle.forward(inp.x, inp.w, h, s, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    assert np.array_equal(bits(y), f32_to_bf16_bits(ref.astype(np.float32)))


@pytest.mark.parametrize("M,K,N,c,BK,BN", [
    (300, 1536, 512, 2, 32, 64),    # 32-wide stages: 256 x 256 tiles, four buffers
    (300, 1536, 384, 2, 96, 64),    # 256 x 128 tiles, a stage at offset 32 of a chunk
    (100, 768, 256, 3, 32, 32),     # 128 x 128 tiles, eight groups per tile
])
def test_fold_32_wide_stages(M, K, N, c, BK, BN):
    wl = Workload("fold32", 9, 2, M, K, N, c, BK, BN, "bf16")
    inp = make_inputs(wl)
    y = run(wl, inp, device_plan(wl), algo="fold")
    check_bf16(wl, inp, y, kernel="fold")
    inp = make_inputs(wl, integer=True)
    y = run(wl, inp, device_plan(wl), algo="fold")
    h, s = oracle_plan(wl)
    ref = oracle.forward(inp.x, inp.w, h, s, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    assert np.array_equal(bits(y), f32_to_bf16_bits(ref.astype(np.float32)))


def test_runs_on_a_side_stream():
    wl = WORKLOADS["gpt2s_up"].with_m(256)
    inp = make_inputs(wl)
    p = device_plan(wl)
    x, w = dev(inp.x_bits, "bf16"), dev(inp.w_bits, "bf16")
    ref = p.forward(x, w)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        y = p.forward(x, w)
    s.synchronize()
    assert torch.equal(ref, y)


# ----------------------------------------------------------- sketch kernel
@pytest.mark.parametrize("name,M", [("gpt2s_up", 40), ("gpt2l_down", 17), ("llama_down_m16", 3),
                                    ("square_c8_bn64", 5), ("tiny", 64)])
def test_sketch_bit_exact(name, M):
    wl = WORKLOADS[name].with_m(M)
    inp = make_inputs(wl)
    p = device_plan(wl)
    h, s = oracle_plan(wl)
    xs = inp.x_bits if wl.dtype == "bf16" else inp.x
    x = dev(xs, wl.dtype)
    z32 = ss1.sketch(x, p.hash, p.sign, wl.c, wl.BK, wl.BN, wl.N)
    torch.cuda.synchronize()
    ref32 = oracle.sketch_rounded(inp.x, h, s, wl.K, wl.N, wl.c, wl.BK, wl.BN, to_bf16=False)
    assert np.array_equal(host(z32).reshape(ref32.shape), ref32)
    if wl.dtype == "bf16":
        zb = ss1.sketch(x, p.hash, p.sign, wl.c, wl.BK, wl.BN, wl.N, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        refb = oracle.sketch_rounded(inp.x, h, s, wl.K, wl.N, wl.c, wl.BK, wl.BN, to_bf16=True)
        assert np.array_equal(host(zb).reshape(refb.shape), refb)


@pytest.mark.parametrize("name", ["gpt2s_up", "gpt2l_up", "gpt2l_down", "llama_gateup_m16", "tiny"])
def test_auto_runs_the_selected_kernel(name):
    wl = WORKLOADS[name].with_m(min(WORKLOADS[name].M, 200))
    algo = ss1.select_algo(wl.M, wl.K, wl.N, wl.c, wl.BK, wl.BN, wl.dtype)
    if name in ("gpt2s_up", "gpt2l_up"):
        assert algo == "band"
    inp = make_inputs(wl)
    p = device_plan(wl)
    assert torch.equal(run(wl, inp, p), run(wl, inp, p, algo=algo))


# ------------------------------------------------- column-split decode (workspace)
def run_ws(wl, inp, plan, workspace=None):
    x = dev(inp.x_bits, "bf16")
    w = dev(inp.w_bits, "bf16")
    y = ss1.forward_ws(x, w, plan.hash, plan.sign, wl.c, wl.BK, wl.BN, workspace=workspace)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("M", [5, 9, 16])
def test_split_llama_decode(M):
    # Llama down: each group's compressed columns split over 4 blocks; float32
    # partial tiles in the workspace, summed in order
    name = "llama_down_m16"
    wl = WORKLOADS[name].with_m(M)
    kernel, nbytes = ss1.forward_ws_query(M, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    assert kernel == "split" and nbytes == 4 * M * wl.N * 4
    inp = make_inputs(wl)
    p = device_plan(wl)
    y = run_ws(wl, inp, p)
    err = check_bf16(wl, inp, y, kernel="split")
    print(f"{name} M={M} split err={err:.3e} workspace={nbytes}", flush=True)


@pytest.mark.parametrize("M,K,N,c,BK,BN", [
    (7, 8192, 512, 4, 64, 32),      # 16 groups -> 16 slices of 128 compressed columns
    (16, 8192, 2048, 2, 64, 64),    # 32 groups -> 8 slices
    (5, 16384, 8192, 2, 128, 64),   # BK = 128: four k-steps per compressed chunk; 4 slices
    (9, 8192, 4096, 1, 64, 64),     # c = 1, 64 groups -> 4 slices
    (6, 6144, 2048, 3, 64, 32),     # c at run time
])
def test_split_shapes(M, K, N, c, BK, BN):
    # input rows too long for the decode kernel (16 rows of K bf16 exceed one
    # block's LDS), so the workspace entry point splits: 16, 8 and 4 slices,
    # c from 1 to 4, BK = 128; against the oracle and bit-exact on integers
    wl = Workload("split_dec", 9, 8, M, K, N, c, BK, BN, "bf16")
    kernel, nbytes = ss1.forward_ws_query(M, K, N, c, BK, BN)
    assert kernel == "split" and nbytes > 0
    p = device_plan(wl)
    inp = make_inputs(wl)
    y = run_ws(wl, inp, p)
    check_bf16(wl, inp, y, kernel="split")
    inp = make_inputs(wl, integer=True)
    y = run_ws(wl, inp, p)
    h, s = oracle_plan(wl)
    ref = oracle.forward(inp.x, inp.w, h, s, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    assert np.array_equal(bits(y), f32_to_bf16_bits(ref.astype(np.float32)))


def test_split_workspace_reused_with_fewer_rows():
    # the workspace's contents on entry are ignored: a second call with fewer
    # rows over the first call's partial sums gives its own result
    wl = WORKLOADS["llama_down_m16"]
    p = device_plan(wl)
    _, nbytes = ss1.forward_ws_query(16, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    for M in (16, 6):
        w = wl.with_m(M)
        inp = make_inputs(w)
        y = run_ws(w, inp, p, workspace=ws)
        check_bf16(w, inp, y, kernel="split")


def test_split_workspace_checks():
    wl = WORKLOADS["llama_down_m16"]
    p = device_plan(wl)
    inp = make_inputs(wl)
    x = dev(inp.x_bits, "bf16")
    w = dev(inp.w_bits, "bf16")
    _, nbytes = ss1.forward_ws_query(wl.M, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    small = torch.empty(nbytes - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ss1.SS1Error) as e:
        ss1.forward_ws(x, w, p.hash, p.sign, wl.c, wl.BK, wl.BN, workspace=small)
    assert e.value.status == 2  # SS1_ERR_SHAPE
    big = torch.empty(nbytes + 64, dtype=torch.uint8, device="cuda")
    with pytest.raises(ss1.SS1Error) as e:
        ss1.forward_ws(x, w, p.hash, p.sign, wl.c, wl.BK, wl.BN, workspace=big[4:])
    assert e.value.status == 5  # SS1_ERR_ALIGN


def test_split_not_applicable_runs_forward():
    # M <= 4 (the matrix-vector kernel) and large M need no workspace and give
    # ss1_forward's bits
    for name, M in (("llama_gateup_m1", 2), ("gpt2s_up", 300)):
        wl = WORKLOADS[name].with_m(M)
        kernel, nbytes = ss1.forward_ws_query(M, wl.K, wl.N, wl.c, wl.BK, wl.BN)
        assert nbytes == 0 and kernel == ss1.select_algo(M, wl.K, wl.N, wl.c, wl.BK, wl.BN, wl.dtype)
        inp = make_inputs(wl)
        p = device_plan(wl)
        assert torch.equal(run_ws(wl, inp, p), run(wl, inp, p))
