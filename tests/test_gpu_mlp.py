"""GPU parity of ss1_mlp_forward (SS1 up-projection, GELU, SS1
down-projection) against the CPU oracle, through the C ABI.

Bars (written in each test):
* h against the mirror of the up-projection kernel that ran (ss1_select_algo:
  bf16-rounded sketch for the sketch kernels, the exact projection for the
  fold kernel) followed by the float64 GELU: |h - ref| <= 2^-7 |ref| +
  1e-5 max|ref| elementwise (one bf16 ulp for h's rounding plus float32
  slack; the device's GELU is within 1.5e-7 absolute), and
  max|h - h64| / max|h64| <= 2e-2 against the float64 chain.
* y against the mirror of the down-projection kernel that ran, applied to the
  device's own h (elementwise as above), and normwise <= 2e-2 against the
  float64 chain with h rounded to bf16.
* row chunks that run the same kernels give bit-identical y; chunkings that
  change the kernel family meet their own kernels' mirrors.
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

    def kernels(self, rows_per_chunk):
        """(up kernel, down kernel) the library runs on a chunk of this many
        rows (ss1_select_algo)."""
        U, D = self.up, self.down
        dt = self.dtype
        return (ss1.select_algo(rows_per_chunk, U["K"], U["N"], U["c"], U["BK"], U["BN"], dt),
                ss1.select_algo(rows_per_chunk, D["K"], D["N"], D["c"], D["BK"], D["BN"], dt))

    def check(self, h, y, rows=None, chunk_rows=None):
        """Normwise bars against the float64 chain, then (bf16) elementwise
        bars against the mirror of each kernel that ran: the sketch kernels
        round the sketch to bf16 (forward_mirror), the fold kernel forms no
        sketch (its mirror is the exact float64 projection).  ``chunk_rows``
        is the row count of the chunk that held these rows (default: all rows
        of the call in one chunk)."""
        x = self.x if rows is None else self.x[rows[0]:rows[1]]
        U, D = self.up, self.down
        bf = self.dtype == "bf16"
        h64, y64 = oracle.mlp_forward(x, U, D, round_h_to_bf16=bf)
        if h is not None:
            assert np.max(np.abs(h - h64)) / np.max(np.abs(h64)) <= (TOL_BF16 if bf else TOL_F32)
        assert np.max(np.abs(y - y64)) / np.max(np.abs(y64)) <= (TOL_BF16 if bf else TOL_F32)
        if not bf:
            return
        ku, kd = self.kernels(chunk_rows or self.M)

        def proj(inp, L, kernel):
            args = (inp, L["Wc"], L["hash"], L["sign"], L["K"], L["N"], L["c"], L["BK"], L["BN"])
            return oracle.forward(*args) if kernel == "fold" else oracle.forward_mirror(*args, True)

        def ulp_ok(got, ref):
            return np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-5 * np.max(np.abs(ref))

        if h is not None:
            ref = oracle.gelu(proj(x, U, ku))
            assert np.all(ulp_ok(h, ref)), f"h off the {ku} mirror"
            ym = proj(h, D, kd)
            assert np.all(ulp_ok(y, ym)), f"y off the {kd} mirror"


def test_mlp_gpt2l_shapes_reduced_rows():
    P = Pair(0x5e00, 300, 1280, 5120, 1280, 4, 4, 64, 64, "bf16")
    h, y = P.run()
    P.check(to_host(h), to_host(y))


def test_mlp_c2_gpt2s_shapes():
    P = Pair(0x5e10, 200, 768, 3072, 768, 2, 2, 64, 64, "bf16")
    h, y = P.run()
    P.check(to_host(h), to_host(y))


def test_mlp_row_chunks_bit_identical():
    # y's bits depend on M only through the kernels each chunk runs: chunks
    # whose kernels (ss1_select_algo) match the whole call's give bit-identical
    # y; other chunkings are held to their own kernels' mirrors
    P = Pair(0x5e20, 300, 1280, 5120, 1280, 4, 4, 64, 64, "bf16")
    _, y_full = P.run()
    whole = P.kernels(300)
    for R in (128, 100, 97, 1):
        h, y = P.run(row_chunk=R)
        assert h.shape[0] == R
        sizes = {R, 300 % R} - {0}
        if all(P.kernels(n) == whole for n in sizes):
            assert torch.equal(y.view(torch.int16), y_full.view(torch.int16)), f"row_chunk {R}"
        yh = to_host(y)
        for r0 in range(0, 300, R):
            n = min(R, 300 - r0)
            P.check(None, yh[r0:r0 + n], rows=(r0, r0 + n), chunk_rows=n)


def test_mlp_row_chunks_change_kernel_family():
    # GPT-2 L pair at 4096 rows: whole, the layers run a large-M kernel; in
    # 9-row chunks they run the small-M kernels.  Sampled rows of each are
    # held elementwise to their own kernels' mirrors (a chunk's h comes from a
    # call on that chunk's rows alone, whose y must be the chunked call's y
    # bit for bit: rows are independent and the kernels are the same).
    P = Pair(0x5e21, 4096, 1280, 5120, 1280, 4, 4, 64, 64, "bf16")
    assert P.kernels(4096) != P.kernels(9)
    assert P.kernels(9) == ("smallm", "smallm")
    hw, yw = P.run()
    _, yc = P.run(row_chunk=9)
    hw, yw = to_host(hw), to_host(yw)
    for r0 in (0, 9 * 227, 4095 - 4095 % 9):
        n = min(9, 4096 - r0)
        P.check(hw[r0:r0 + n], yw[r0:r0 + n], rows=(r0, r0 + n), chunk_rows=4096)
        h9, y9 = P.run(rows=(r0, r0 + n))
        assert torch.equal(y9.view(torch.int16), yc[r0:r0 + n].view(torch.int16))
        P.check(to_host(h9), to_host(y9), rows=(r0, r0 + n), chunk_rows=n)


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


@pytest.mark.parametrize("c_up,kernels", [(4, ("fold", "fold")), (2, ("fold", "fold"))])
def test_mlp_full_size_sampled_rows(c_up, kernels):
    # the GPT-2 L pair at 8192 rows in one chunk (the bench's setting): both
    # projections run the fold kernel, the up-projection with the GELU
    # epilogue; sampled rows of h and y are held elementwise to the mirrors of
    # the kernels that ran
    P = Pair(0x5e60, 8192, 1280, 5120, 1280, c_up, 4, 64, 64, "bf16")
    assert P.kernels(8192) == kernels
    h, y = P.run(row_chunk=8192)
    h, y = to_host(h), to_host(y)
    for r0 in (0, 4093, 8184):
        P.check(h[r0:r0 + 8], y[r0:r0 + 8], rows=(r0, r0 + 8), chunk_rows=8192)
    # in 2048-row chunks (h then stays in the last-level cache)
    _, y = P.run(row_chunk=2048)
    y = to_host(y)
    for r0 in (0, 4093, 8184):
        P.check(None, y[r0:r0 + 8], rows=(r0, r0 + 8), chunk_rows=2048)


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
