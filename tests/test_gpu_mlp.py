"""GPU parity of ss1_mlp_forward (SS1 up-projection, GELU, SS1
down-projection) against the CPU oracle, through the C ABI.

Bars (written in each test):
* h against the oracle's float32 mirror of the up-projection followed by the
  float64 GELU: |h - ref| <= 2^-7 |ref| + 1e-5 max|ref| elementwise (one bf16
  ulp for h's rounding plus float32 slack; the device's erff is within a few
  float32 ulp), and max|h - h64| / max|h64| <= 2e-2 against the float64 chain.
* y against the oracle's mirror of the down-projection applied to the
  device's own h (elementwise as above), and normwise <= 2e-2 against the
  float64 chain with h rounded to bf16.
* row chunks that run the same kernels give bit-identical y.
* float32 layers: normwise <= 1e-5 against the float64 chain.
"""
import numpy as np
import pytest

import oracle
import sketched_parameter_sharing_amd as ss1
from ss1_inputs import Workload, bf16_bits_to_f32, draw, f32_to_bf16_bits

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
TOL_F32 = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ss1.load()


def to_dev(a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(f32_to_bf16_bits(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def exact_values(a, dtype):
    return bf16_bits_to_f32(f32_to_bf16_bits(a)).astype(np.float64) if dtype == "bf16" else \
        np.asarray(a, dtype=np.float32).astype(np.float64)


def to_host(t):
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


class Pair:
    """An up (K -> N1) and down (N1 -> N2) SS1 layer with seeded weights."""

    def __init__(self, seed, M, K, N1, N2, c1, c2, BK, BN, dtype):
        self.M, self.dtype = M, dtype
        self.up = dict(K=K, N=N1, c=c1, BK=BK, BN=BN)
        self.down = dict(K=N1, N=N2, c=c2, BK=BK, BN=BN)
        self.x32 = draw("normal", seed, (M, K))
        self.dev = {}
        for name, L, s in (("up", self.up, seed + 1), ("down", self.down, seed + 2)):
            w32 = draw("normal002", s, (L["N"], L["K"] // L["c"]))
            L["Wc"] = exact_values(w32, dtype)
            L["hash"], L["sign"] = oracle.plan(s, L["K"], L["N"], L["c"], L["BK"], L["BN"])
            p = ss1.DevicePlan.make(s, L["K"], L["N"], L["c"], L["BK"], L["BN"])
            self.dev[name] = (to_dev(w32, dtype), p.hash, p.sign, L["c"], L["BK"], L["BN"])
        self.x = exact_values(self.x32, dtype)
        self.xd = to_dev(self.x32, dtype)

    def run(self, rows=None, row_chunk=None):
        xd = self.xd if rows is None else self.xd[rows[0]:rows[1]]
        h, y = ss1.mlp_forward(xd, self.dev["up"], self.dev["down"], row_chunk=row_chunk)
        torch.cuda.synchronize()
        return h, y

    def check(self, h, y, rows=None):
        x = self.x if rows is None else self.x[rows[0]:rows[1]]
        U, D = self.up, self.down
        bf = self.dtype == "bf16"
        h64, y64 = oracle.mlp_forward(x, U, D, round_h_to_bf16=bf)
        if h is not None:
            assert np.max(np.abs(h - h64)) / np.max(np.abs(h64)) <= (TOL_BF16 if bf else TOL_F32)
        assert np.max(np.abs(y - y64)) / np.max(np.abs(y64)) <= (TOL_BF16 if bf else TOL_F32)
        if not bf:
            return
        if h is not None:
            a = oracle.forward_mirror(x, U["Wc"], U["hash"], U["sign"], U["K"], U["N"], U["c"], U["BK"],
                                      U["BN"], True)
            ref = oracle.gelu(a)
            assert np.all(np.abs(h - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-5 * np.max(np.abs(ref)))
            ym = oracle.forward_mirror(h, D["Wc"], D["hash"], D["sign"], D["K"], D["N"], D["c"], D["BK"],
                                       D["BN"], True)
            assert np.all(np.abs(y - ym) <= 2.0 ** -7 * np.abs(ym) + 1e-5 * np.max(np.abs(ym)))


def test_mlp_gpt2l_shapes_reduced_rows():
    P = Pair(0x5e00, 300, 1280, 5120, 1280, 4, 4, 64, 64, "bf16")
    h, y = P.run()
    P.check(to_host(h), to_host(y))


def test_mlp_c2_gpt2s_shapes():
    P = Pair(0x5e10, 200, 768, 3072, 768, 2, 2, 64, 64, "bf16")
    h, y = P.run()
    P.check(to_host(h), to_host(y))


def test_mlp_row_chunks_bit_identical():
    # chunks of more than 16 rows run the same kernels as the whole call, whose
    # per-output arithmetic does not depend on the row count
    P = Pair(0x5e20, 300, 1280, 5120, 1280, 4, 4, 64, 64, "bf16")
    _, y_full = P.run()
    for R in (128, 100):
        h, y = P.run(row_chunk=R)
        assert h.shape[0] == R
        assert torch.equal(y.view(torch.int16), y_full.view(torch.int16)), f"row_chunk {R}"
    # a last chunk of 9 rows, and one row per chunk, take the small-M kernels
    for R in (97, 1):
        _, y = P.run(row_chunk=R)
        P.check(None, to_host(y))


def test_mlp_small_m_and_odd_shapes():
    P = Pair(0x5e30, 7, 512, 384, 256, 2, 4, 32, 32, "bf16")
    h, y = P.run()
    P.check(to_host(h), to_host(y))
    P = Pair(0x5e40, 70, 240, 96, 48, 2, 2, 24, 48, "bf16")   # generic kernels (BK % 32 != 0)
    h, y = P.run()
    P.check(to_host(h), to_host(y))


def test_mlp_decode_matrix_vector():
    # M <= 4 with compressed rows of 1024: both layers run the matrix-vector
    # kernel, the up-projection with GELU in its epilogue
    for M in (1, 3):
        P = Pair(0x5e60 + M, M, 2048, 1024, 512, 2, 1, 64, 64, "bf16")
        assert ss1.select_algo(M, 2048, 1024, 2, 64, 64) == "gemv"
        assert ss1.select_algo(M, 1024, 512, 1, 64, 64) == "gemv"
        h, y = P.run()
        P.check(to_host(h), to_host(y))


def test_mlp_float32_tiny():
    P = Pair(0x5e50, 64, 256, 256, 128, 2, 2, 32, 32, "f32")
    h, y = P.run()
    P.check(to_host(h), to_host(y))


def test_mlp_full_size_sampled_rows():
    P = Pair(0x5e60, 8192, 1280, 5120, 1280, 4, 4, 64, 64, "bf16")
    _, y = P.run(row_chunk=2048)
    y = to_host(y)
    for r0 in (0, 4093, 8184):
        P.check(None, y[r0:r0 + 8], rows=(r0, r0 + 8))


def test_mlp_empty_and_no_write_past_end():
    P = Pair(0x5e70, 96, 768, 3072, 768, 2, 2, 64, 64, "bf16")
    e = torch.empty((0, 768), dtype=torch.bfloat16, device="cuda")
    h, y = ss1.mlp_forward(e, P.dev["up"], P.dev["down"], h=torch.empty((4, 3072), dtype=torch.bfloat16,
                                                                        device="cuda"))
    assert y.shape == (0, 768)
    buf = torch.full((96 * 768 + 64,), 777, dtype=torch.int16, device="cuda")
    yv = buf[:96 * 768].view(torch.bfloat16).view(96, 768)
    ss1.mlp_forward(P.xd, P.dev["up"], P.dev["down"], y=yv, row_chunk=40)
    torch.cuda.synchronize()
    assert torch.all(buf[96 * 768:] == 777)
    P.check(None, to_host(yv))
