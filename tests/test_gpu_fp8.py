"""GPU parity of the fp8-weight path (ss1_quantize_fp8, ss1_forward_fp8w)
against the CPU oracle, through the C ABI.

Bars (written in each test):
* quantization: codes and float32 scales bit-exact against the oracle's
  quantize_fp8_rows (which is pinned against torch's float8_e4m3fn);
* forward: the layer with W_c = e4m3(Q) * scale; against the float64 oracle
  max|y - y_ref| / max|y_ref| <= 2e-2, and elementwise against the oracle's
  mirror of the kernel that ran, |y - y_m| <= 2^-7 |y_m| + 1e-5 max|y_m|:
  the bf16-rounded sketch followed by a float64 contraction for the sketch
  kernels, the float64 result itself for the fold kernel (which forms no
  sketch) -- the same bars as the bf16 path, since every E4M3 weight is a
  bf16 value and only the row scale's float32 product is added.
"""
import numpy as np
import pytest

import oracle
import sketched_parameter_sharing_amd as ss1
from ss1_inputs import WORKLOADS, Workload, bf16_bits_to_f32, draw, f32_to_bf16_bits, make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ss1.load()


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_host(t):
    return bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)


@pytest.mark.parametrize("N,Kc,dtype", [(64, 128, "bf16"), (130, 384, "bf16"), (96, 2048, "f32"),
                                        (3, 2, "bf16"), (14336, 2048, "bf16"), (7, 4096, "bf16"),
                                        (5, 4104, "bf16"), (2, 16384, "bf16"), (3, 20000, "f32")])
def test_quantize_bit_exact(N, Kc, dtype):
    # rows of a multiple of 8 elements: one block per row with up to 16384
    # elements in registers (20000: the rest read twice); other lengths the
    # scalar kernel
    w = draw("normal002", 0x5800 + N + Kc, (N, Kc))
    w[min(1, N - 1)] = 0.0                        # an all-zero row
    if N > 2:
        w[2, ::7] *= 300.0                        # a row with outliers
    if dtype == "bf16":
        bits = f32_to_bf16_bits(w)
        vals = bf16_bits_to_f32(bits)
        W = bf16_dev(bits)
    else:
        vals = w
        W = torch.from_numpy(w).cuda()
    Q, scale = ss1.quantize_fp8(W)
    torch.cuda.synchronize()
    codes, sc = oracle.quantize_fp8_rows(vals)
    assert np.array_equal(scale.cpu().numpy().view(np.uint32), sc.view(np.uint32))
    assert np.array_equal(Q.cpu().numpy(), codes)


def run_case(wl, M, rows=None):
    inp = make_inputs(wl.with_m(M))
    p = ss1.DevicePlan.make(wl.plan_seed, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    Q, scale = ss1.quantize_fp8(bf16_dev(inp.w_bits))
    y = ss1.forward_fp8w(bf16_dev(inp.x_bits), Q, scale, p.hash, p.sign, wl.c, wl.BK, wl.BN)
    torch.cuda.synchronize()
    y = to_host(y)
    h, s = oracle.plan(wl.plan_seed, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    Wq = oracle.dequantize_fp8_rows(Q.cpu().numpy(), scale.cpu().numpy())
    x = inp.x.astype(np.float64)
    if rows is not None:
        x, y = x[rows], y[rows]
    ref = oracle.forward(x, Wq, h, s, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    assert np.max(np.abs(y - ref)) / np.max(np.abs(ref)) <= 2e-2
    # one bf16 ulp of the mirror of the kernel that ran (the library reports
    # it): the sketch kernels round the sketch to bf16 first; the fold kernel
    # (large M) forms no sketch, so its mirror is the exact result
    kernel = ss1.select_algo(M, wl.K, wl.N, wl.c, wl.BK, wl.BN, weights="fp8")
    if kernel == "fold":
        mir = ref
    else:
        mir = oracle.forward_mirror(x, Wq, h, s, wl.K, wl.N, wl.c, wl.BK, wl.BN, True)
    bad = np.abs(y - mir) > 2.0 ** -7 * np.abs(mir) + 1e-5 * np.max(np.abs(mir))
    assert not bad.any(), f"{wl.name} M={M} ({kernel}): {int(bad.sum())} outputs off the mirror"
    return kernel


@pytest.mark.parametrize("M", [1, 3, 5, 16, 300])
@pytest.mark.parametrize("c,BN", [(1, 64), (2, 64), (4, 32), (8, 128), (3, 64)])
def test_forward_fp8w_reduced(M, c, BN):
    K = 96 * 64 if c == 3 else 2048
    wl = Workload(f"fp8_c{c}_bn{BN}", 8, c, M, K, 4 * BN, c, 64, BN, "bf16")
    run_case(wl, M)


def test_forward_fp8w_decode_bn48_and_ragged():
    wl = Workload("fp8_bn48", 8, 9, 7, 768, 3 * 48, 2, 32, 48, "bf16")   # small-M kernel only
    run_case(wl, 7)
    wl = Workload("fp8_ragged", 8, 10, 333, 768, 6 * 64, 2, 32, 64, "bf16")
    run_case(wl, 333)


@pytest.mark.parametrize("M,K,N,c,BK,BN", [
    (1, 32768, 32, 2, 64, 16),      # two 8-weight slices per thread, 1024 threads
    (2, 65536, 32, 2, 64, 32),      # four slices per thread, two tokens
    (4, 16384, 64, 4, 64, 16),      # four token slots, 512 threads
    (3, 6144, 96, 3, 64, 48),       # c at run time
])
def test_forward_fp8w_matrix_vector(M, K, N, c, BK, BN):
    assert ss1.select_algo(M, K, N, c, BK, BN, weights="fp8") == "gemv"
    run_case(Workload("fp8_gemv", 8, 12, M, K, N, c, BK, BN, "bf16"), M)


def test_forward_fp8w_fold_shape():
    # a large-M layer that the library runs on the fold kernel (E4M3 weight
    # tile widened to bf16 as it leaves LDS), with a ragged last row tile
    wl = Workload("fp8_fold", 8, 11, 4000, 2048, 4096, 2, 64, 64, "bf16")
    assert run_case(wl, wl.M, np.r_[0:8, 1999:2007, 3990:4000]) == "fold"


@pytest.mark.parametrize("name", ["llama_gateup_m1", "llama_gateup_m16", "llama_down_m16", "gpt2s_up",
                                  "llama_gateup_m4096", "gpt2l_down"])
def test_forward_fp8w_full_size(name):
    # gpt2l_down runs the fold on 192-token tiles with E4M3 weights (three
    # stages); its last row tile holds 128 rows
    wl = WORKLOADS[name]
    rows = None
    if wl.M > 16:
        rows = np.r_[0:4, 191:193, wl.M // 2:wl.M // 2 + 4, 8063:8065, wl.M - 4:wl.M]
        rows = np.unique(rows[rows < wl.M])
    run_case(wl, wl.M, rows)


# ------------------------------------------- fp8 input and weights (fp8 MFMA)
# ss1_forward_fp8: x and W_c both E4M3 with per-row scales, contracted on the
# fp8 matrix cores.  The layer it computes is SS1 of the dequantized operands;
# the kernel forms no sketch (fold) and every product of two E4M3 values is
# exact in float32, so the mirror is the float64 oracle of the dequantized
# layer, under one bf16 ulp plus the float32 summation bound (below).  Integer
# codes with power-of-two scales make every sum exact: y must then equal the
# rounded oracle bit for bit.

def e4m3_int_codes(g, shape):
    """E4M3 codes of integers in {-4..4} (exact in E4M3)."""
    vals = g.integers(-4, 5, shape)
    lut = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48}
    codes = np.vectorize(lambda v: lut[abs(v)] | (0x80 if v < 0 else 0))(vals).astype(np.uint8)
    return codes, vals.astype(np.float64)


def rne_bf16(a):
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(a, dtype=np.float32))).astype(np.float64)


@pytest.mark.parametrize("M,K,N,c,BK,BN", [(300, 2048, 512, 2, 64, 64), (257, 1024, 256, 4, 64, 32),
                                           (40, 4096, 256, 1, 128, 128), (513, 768, 768, 2, 64, 256)])
def test_forward_fp8_integer_bit_exact(M, K, N, c, BK, BN):
    g = np.random.default_rng(M + K)
    xc, xv = e4m3_int_codes(g, (M, K))
    wc, wv = e4m3_int_codes(g, (N, K // c))
    xs = (2.0 ** g.integers(-2, 3, M)).astype(np.float32)
    wsc = (2.0 ** g.integers(-2, 3, N)).astype(np.float32)
    p = ss1.DevicePlan.make(0x8100 + M, K, N, c, BK, BN)
    y = ss1.forward_fp8(torch.from_numpy(xc).cuda(), torch.from_numpy(xs).cuda(), torch.from_numpy(wc).cuda(),
                        torch.from_numpy(wsc).cuda(), p.hash, p.sign, c, BK, BN)
    torch.cuda.synchronize()
    h, s = oracle.plan(0x8100 + M, K, N, c, BK, BN)
    ref = oracle.forward(xv * xs[:, None], wv * wsc[:, None], h, s, K, N, c, BK, BN)
    assert np.array_equal(to_host(y), rne_bf16(ref))


def run_fp8a(wl, M, rows=None):
    """Quantize x and W_c on the device, run ss1_forward_fp8, check against the
    dequantized layer's float64 oracle (the mirror) and report the error
    against the unquantized bf16 layer."""
    inp = make_inputs(wl.with_m(M))
    p = ss1.DevicePlan.make(wl.plan_seed, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    xq, xs = ss1.quantize_fp8(bf16_dev(inp.x_bits))
    Q, wsc = ss1.quantize_fp8(bf16_dev(inp.w_bits))
    y = ss1.forward_fp8(xq, xs, Q, wsc, p.hash, p.sign, wl.c, wl.BK, wl.BN)
    torch.cuda.synchronize()
    y = to_host(y)
    h, s = oracle.plan(wl.plan_seed, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    codes_x, sc_x = xq.cpu().numpy(), xs.cpu().numpy()
    if rows is not None:
        codes_x, sc_x, y, x = codes_x[rows], sc_x[rows], y[rows], inp.x[rows]
    else:
        x = inp.x
    # the device quantizer is the oracle's (codes and scales bit for bit)
    qc, qs = oracle.quantize_fp8_rows(x)
    assert np.array_equal(codes_x, qc) and np.array_equal(sc_x.view(np.uint32), qs.view(np.uint32))
    xd = oracle.dequantize_fp8_rows(codes_x, sc_x)
    Wd = oracle.dequantize_fp8_rows(Q.cpu().numpy(), wsc.cpu().numpy())
    ref = oracle.forward(xd, Wd, h, s, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    # bar: one bf16 ulp of the result, plus the worst case of a float32 sum of
    # K exact products in any order (K * 2^-24 * sum of |products|, Higham's
    # bound), plus the two float32 scale multiplies; a float32 sum of K = 2048
    # to 14336 products can leave an output that nearly cancels well outside
    # 1e-5 max|y|, which no rounding-order-free bar can exclude
    sum_abs = np.abs(xd) @ np.abs(oracle.dense_expand(Wd, h, s, wl.K, wl.N, wl.c, wl.BK, wl.BN)).T
    bound = 2.0 ** -7 * np.abs(ref) + wl.K * 2.0 ** -24 * sum_abs + 2.0 ** -22 * np.abs(ref)
    bad = np.abs(y - ref) > bound
    assert not bad.any(), f"{wl.name}: {int(bad.sum())} outputs off the dequantized layer beyond the bar"
    # and the bf16 bar the other kernels meet, on all but a few near-cancelling outputs
    tight = np.abs(y - ref) > 2.0 ** -7 * np.abs(ref) + 1e-5 * np.max(np.abs(ref))
    assert tight.sum() <= max(1, tight.size // 10000)
    # against the unquantized layer: E4M3 keeps 3 mantissa bits (relative
    # rounding error <= 2^-4 per operand), so each product is off by about
    # 2^-3 relative at most and the errors of K random-signed terms add like
    # a random walk: normwise (by max|y|) error well under 5e-2
    full = oracle.forward(x, inp.w, h, s, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    err = np.max(np.abs(y - full)) / np.max(np.abs(full))
    assert err <= 5e-2, f"{wl.name}: error against the bf16 layer {err:.3e}"
    return err


def test_forward_fp8_reduced_ragged():
    wl = Workload("fp8a_ragged", 8, 31, 300, 2048, 512, 2, 64, 64, "bf16")
    run_fp8a(wl, 300)


@pytest.mark.parametrize("name", ["llama_gateup_m4096", "llama_down_m4096", "gpt2l_up", "gpt2l_down", "gpt2s_up"])
def test_forward_fp8_full_size_sampled(name):
    wl = WORKLOADS[name]
    rows = np.r_[0:4, 255:257, wl.M // 2:wl.M // 2 + 4, wl.M - 4:wl.M]
    run_fp8a(wl, wl.M, rows)
