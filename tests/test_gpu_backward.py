"""GPU parity of ss1_backward (dx and dW_c) against the CPU oracle, through
the C ABI.

Bars (written in each test):
* integer-valued x, W_c and dy in {-4..4}: the sketch is exact in bf16 and
  every float32 sum is an exact integer below 2^24, so dx and dW_c equal the
  float64 oracle rounded to bf16 (nearest even) bit for bit;
* random inputs: max|d - d_ref| / max|d_ref| <= 2e-2 against the float64
  oracle, and elementwise |d - d_m| <= 2^-7 |d_m| + 1e-5 max|d_m| against
  the mirror of the kernel the library reports (ss1_backward_select_algo):
  dW_c from the bf16-rounded sketch for the sketch kernel, the float64 oracle
  itself for the fold kernel (no sketch formed); dx has no sketch rounding on
  either kernel, so its mirror is the float64 oracle itself.
"""
import numpy as np
import pytest

import oracle
import sketched_parameter_sharing_amd as ss1
from ss1_inputs import WORKLOADS, bf16_bits_to_f32, draw, f32_to_bf16_bits

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ss1.load()


def dev(a):
    return torch.from_numpy(f32_to_bf16_bits(a).view(np.int16)).view(torch.bfloat16).cuda()


def exact(a):
    return bf16_bits_to_f32(f32_to_bf16_bits(a)).astype(np.float64)


def host(t):
    return bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)


def rne_bf16(a):
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(a, dtype=np.float32))).astype(np.float64)


def inputs(seed, M, K, N, c, integer):
    dist_x, dist_w = ("int4", "int4") if integer else ("normal", "normal002")
    return (draw(dist_x, seed, (M, K)), draw(dist_w, seed + 1, (N, K // c)),
            draw("int4" if integer else "normal", seed + 2, (M, N)))


def run(seed, M, K, N, c, BK, BN, want_dx=True, want_dw=True, integer=False):
    x, w, dy = inputs(seed, M, K, N, c, integer)
    p = ss1.DevicePlan.make(seed, K, N, c, BK, BN)
    dx, dw = ss1.backward(dev(x), dev(w), p.hash, p.sign, c, BK, BN, dev(dy),
                          dx=True if want_dx else None, dW_c=True if want_dw else None)
    torch.cuda.synchronize()
    h, s = oracle.plan(seed, K, N, c, BK, BN)
    return (exact(x), exact(w), exact(dy), h, s,
            host(dx) if dx is not None else None, host(dw) if dw is not None else None)


def within_ulp(got, mirror):
    return np.abs(got - mirror) <= 2.0 ** -7 * np.abs(mirror) + 1e-5 * np.max(np.abs(mirror))


def check_close(got, ref, mirror):
    """Normwise against the float64 oracle, then elementwise within one bf16
    ulp of the mirror of the kernel that ran."""
    assert np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30) <= 2e-2
    bad = ~within_ulp(got, mirror)
    assert not bad.any(), f"{int(bad.sum())} outputs off the mirror by more than one bf16 ulp"


def dw_mirror(x, dy, h, s, rdw, layer, K, N, c, BK, BN):
    """Mirror of the dW_c kernel the library reports for ``layer`` (its
    (M, K, N, c, BK, BN)): the sketch kernel contracts the bf16-rounded sketch
    (backward_dw_mirror over the given K, N and plan rows); the fold kernel
    forms no sketch, so its mirror is the exact float64 result ``rdw``."""
    _, dw_kernel = ss1.backward_select_algo(*layer)
    if dw_kernel == "fold":
        return rdw
    assert dw_kernel == "fused"
    return oracle.backward_dw_mirror(x, dy, h, s, K, N, c, BK, BN)


SHAPES = [  # M, K, N, c, BK, BN
    (300, 768, 192, 2, 64, 64), (100, 512, 128, 1, 64, 32), (257, 1024, 256, 4, 32, 128),
    (64, 576, 96, 3, 64, 32), (130, 2048, 64, 8, 64, 64),
    (200, 4096, 128, 2, 64, 64), (72, 3072, 64, 3, 64, 32),   # Kc >= 1024 (wide dW tiles)
    (50, 1280, 128, 1, 160, 32), (40, 384, 96, 2, 96, 32),    # chunks that straddle 128-column dx tiles
    (150, 1024, 256, 2, 128, 64), (90, 512, 256, 2, 64, 128),  # dx fold: 64-feature tiles inside 128-wide chunks; BN = 128
    (4096, 4096, 128, 2, 64, 64)]   # dx fold with 256-token tiles


@pytest.mark.parametrize("M,K,N,c,BK,BN", SHAPES)
def test_backward_integer_bit_exact(M, K, N, c, BK, BN):
    x, w, dy, h, s, dx, dw = run(0x4b00 + M, M, K, N, c, BK, BN, integer=True)
    rdx, rdw = oracle.backward(x, w, dy, h, s, K, N, c, BK, BN)
    assert np.array_equal(dx, rne_bf16(rdx))
    assert np.array_equal(dw, rne_bf16(rdw))


@pytest.mark.parametrize("M,K,N,c,BK,BN", SHAPES)
def test_backward_random(M, K, N, c, BK, BN):
    x, w, dy, h, s, dx, dw = run(0x4c00 + M, M, K, N, c, BK, BN)
    rdx, rdw = oracle.backward(x, w, dy, h, s, K, N, c, BK, BN)
    check_close(dx, rdx, rdx)
    check_close(dw, rdw, dw_mirror(x, dy, h, s, rdw, (M, K, N, c, BK, BN), K, N, c, BK, BN))


def test_backward_one_output_only_and_empty():
    M, K, N, c, BK, BN = 96, 512, 128, 2, 64, 64
    _, _, _, _, _, dx, dw = run(0x4d00, M, K, N, c, BK, BN, want_dw=False)
    assert dw is None and dx.shape == (M, K)
    _, _, _, _, _, dx, dw = run(0x4d00, M, K, N, c, BK, BN, want_dx=False)
    assert dx is None and dw.shape == (N, K // c)
    # M = 0: dW_c is a sum over no tokens
    p = ss1.DevicePlan.make(1, K, N, c, BK, BN)
    e = torch.empty((0, K), dtype=torch.bfloat16, device="cuda")
    dW = torch.full((N, K // c), 3.0, dtype=torch.bfloat16, device="cuda")
    ss1.backward(e, dev(np.ones((N, K // c), np.float32)), p.hash, p.sign, c, BK, BN,
                 torch.empty((0, N), dtype=torch.bfloat16, device="cuda"), dx=None, dW_c=dW)
    torch.cuda.synchronize()
    assert not dW.float().any()


def test_backward_full_size_sampled():
    wl = WORKLOADS["gpt2s_up"]
    M, K, N, c, BK, BN = wl.M, wl.K, wl.N, wl.c, wl.BK, wl.BN
    assert ss1.backward_select_algo(M, K, N, c, BK, BN) == ("fold", "fold")
    x, w, dy, h, s, dx, dw = run(0x4e00, M, K, N, c, BK, BN)
    rows = np.r_[0:4, M // 2:M // 2 + 4, M - 4:M]
    W = oracle.dense_expand(w, h, s, K, N, c, BK, BN)
    rdx = dy[rows] @ W
    check_close(dx[rows], rdx, rdx)
    groups = [0, 23, wl.G - 1]
    cols = np.concatenate([np.arange(g * BN, (g + 1) * BN) for g in groups])
    hs, ss = h[groups], s[groups]
    Ns = len(groups) * BN
    z = oracle.sketch(x, hs, ss, K, Ns, c, BK, BN)
    ref = np.concatenate([dy[:, cols[i * BN:(i + 1) * BN]].T @ z[i] for i in range(len(groups))])
    check_close(dw[cols], ref, dw_mirror(x, dy[:, cols], hs, ss, ref, (M, K, N, c, BK, BN), K, Ns, c, BK, BN))


def test_backward_full_size_sampled_gpt2l_down():
    # the combined dW_c + dx fold launch on a c = 4 layer with long rows: 200
    # dW_c tiles (64 neurons x 128 compressed columns) and 128-token dx tiles
    wl = WORKLOADS["gpt2l_down"]
    M, K, N, c, BK, BN = wl.M, wl.K, wl.N, wl.c, wl.BK, wl.BN
    assert ss1.backward_select_algo(M, K, N, c, BK, BN) == ("fold", "fold")
    x, w, dy, h, s, dx, dw = run(0x4f00, M, K, N, c, BK, BN)
    rows = np.r_[0:4, M // 2:M // 2 + 4, M - 4:M]
    W = oracle.dense_expand(w, h, s, K, N, c, BK, BN)
    rdx = dy[rows] @ W
    check_close(dx[rows], rdx, rdx)
    groups = [0, 9, wl.G - 1]
    cols = np.concatenate([np.arange(g * BN, (g + 1) * BN) for g in groups])
    hs, ss = h[groups], s[groups]
    Ns = len(groups) * BN
    z = oracle.sketch(x, hs, ss, K, Ns, c, BK, BN)
    ref = np.concatenate([dy[:, cols[i * BN:(i + 1) * BN]].T @ z[i] for i in range(len(groups))])
    check_close(dw[cols], ref, dw_mirror(x, dy[:, cols], hs, ss, ref, (M, K, N, c, BK, BN), K, Ns, c, BK, BN))
