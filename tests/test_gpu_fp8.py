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
                                        (3, 2, "bf16"), (14336, 2048, "bf16")])
def test_quantize_bit_exact(N, Kc, dtype):
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
