"""GPU parity of ss1_project (least-squares projection of a dense weight onto
the SS1 sharing pattern) against the CPU oracle, through the C ABI.

Bars (written in each test):
* every case is bit-exact against the oracle's float32 mirror
  (``project_rounded``: ascending float32 sum of the signed sources, IEEE
  division by c, bf16 rounding to nearest even for bf16 weights), and within
  one bf16 half-ulp (2^-9 relative, plus float32 slack) of the float64 oracle;
* at full layer sizes the sampled groups are bit-exact against the mirror, and
  projecting an SS1 layer's own dense expansion returns its weights bit for
  bit (the sum of c copies of +-w is exact in float32 and the division by a
  power of two is exact).
"""
import numpy as np
import pytest

import oracle
import sketched_parameter_sharing_amd as ss1
from ss1_inputs import WORKLOADS, Workload, bf16_bits_to_f32, draw, f32_to_bf16_bits, make_dense_weight

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ss1.load()


def to_dev(values, bits, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(values, dtype=np.float32)).cuda()


def to_host(t):
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def project_gpu(wl, W_dev):
    p = ss1.DevicePlan.make(wl.plan_seed, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    out = ss1.project(W_dev, p.hash, p.sign, wl.c, wl.BK, wl.BN)
    torch.cuda.synchronize()
    return out


def check(wl, got, W_vals, groups=None):
    h, s = oracle.plan(wl.plan_seed, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    if groups is not None:   # a subset of groups: a smaller layer with their rows and plans
        rows = np.concatenate([np.arange(g * wl.BN, (g + 1) * wl.BN) for g in groups])
        W_vals, got, h, s = W_vals[rows], got[rows], h[groups], s[groups]
        N = len(groups) * wl.BN
    else:
        N = wl.N
    mirror = oracle.project_rounded(W_vals, h, s, wl.K, N, wl.c, wl.BK, wl.BN, wl.dtype == "bf16")
    assert np.array_equal(got, mirror), "not bit-exact against the float32 mirror"
    exact = oracle.project(W_vals, h, s, wl.K, N, wl.c, wl.BK, wl.BN)
    # float32 sum: at most c roundings of 2^-24 of the running |sum|, bounded by
    # the mean |source| times c; then one output rounding (bf16: 2^-8 relative)
    abs_mean = oracle.project(np.abs(W_vals), h, np.ones_like(s), wl.K, N, wl.c, wl.BK, wl.BN)
    rel = 2.0 ** -8 if wl.dtype == "bf16" else 2.0 ** -23
    bound = rel * np.abs(exact) + 2 * wl.c * 2.0 ** -24 * abs_mean * wl.c
    assert np.all(np.abs(got - exact) <= bound)


CASES = [  # name, K, N, c, BK, BN, dtype
    ("f32_tiny", 256, 256, 2, 32, 32, "f32"),
    ("f32_c3_runtime", 384, 96, 3, 32, 32, "f32"),
    ("bf16_c1", 512, 192, 1, 64, 64, "bf16"),
    ("bf16_c2", 768, 320, 2, 64, 64, "bf16"),
    ("bf16_c4", 1280, 5 * 40, 4, 64, 40, "bf16"),
    ("bf16_ragged_row_slices", 4096, 3 * 40, 2, 64, 40, "bf16"),
    ("bf16_c8", 2048, 128, 8, 64, 128, "bf16"),
    ("bf16_c2_long_rows", 4096, 3 * 128, 2, 64, 128, "bf16"),
    ("bf16_bk8_bn3", 96, 3 * 7, 2, 8, 3, "bf16"),
    ("bf16_c3_runtime", 576, 48, 3, 64, 16, "bf16"),
    ("bf16_one_group_one_chunk", 128, 64, 2, 64, 64, "bf16"),
    ("f32_bk4", 64, 10, 2, 4, 5, "f32"),
]


@pytest.mark.parametrize("name,K,N,c,BK,BN,dtype", CASES, ids=[c[0] for c in CASES])
def test_project_bit_exact_against_mirror(name, K, N, c, BK, BN, dtype):
    wl = Workload("proj_" + name, 9, len(name), 0, K, N, c, BK, BN, dtype)
    vals, bits = make_dense_weight(wl)
    got = to_host(project_gpu(wl, to_dev(vals, bits, dtype)))
    check(wl, got, vals.astype(np.float64))


@pytest.mark.parametrize("name,K,N,c,BK,BN,dtype", CASES[:6], ids=[c[0] for c in CASES[:6]])
def test_project_integer_inputs_exact(name, K, N, c, BK, BN, dtype):
    wl = Workload("proj_" + name, 9, len(name), 0, K, N, c, BK, BN, dtype)
    vals, bits = make_dense_weight(wl, integer=True)
    got = to_host(project_gpu(wl, to_dev(vals, bits, dtype)))
    check(wl, got, vals.astype(np.float64))


@pytest.mark.parametrize("name", ["llama_gateup_m1", "llama_down_m1", "gpt2s_up"])
def test_project_full_size_sampled_groups(name):
    wl = WORKLOADS[name]
    vals, bits = make_dense_weight(wl)
    got = to_host(project_gpu(wl, to_dev(vals, bits, wl.dtype)))
    check(wl, got, vals.astype(np.float64), groups=[0, 1, wl.G // 2, wl.G - 1])


@pytest.mark.parametrize("name", ["llama_gateup_m1", "gpt2l_down"])
def test_project_of_expansion_returns_the_layer(name):
    """Property at full size: W = dense expansion of an SS1 layer, expanded
    on the GPU by indexing with the plan; projecting it returns W_c exactly."""
    wl = WORKLOADS[name]
    p = ss1.DevicePlan.make(wl.plan_seed, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    wc_bits = f32_to_bf16_bits(draw("normal002", wl.w_seed, (wl.N, wl.Kc)))
    Wc = torch.from_numpy(wc_bits.view(np.int16)).view(torch.bfloat16).cuda()
    hash_ = p.hash.long()                               # [G][J]
    sign = p.sign.to(torch.float32)                     # [G][J]
    Wc3 = Wc.float().view(wl.G, wl.BN, wl.Jc, wl.BK)
    idx = hash_.view(wl.G, 1, wl.J, 1).expand(wl.G, wl.BN, wl.J, wl.BK)
    W = torch.gather(Wc3, 2, idx) * sign.view(wl.G, 1, wl.J, 1)
    W = W.reshape(wl.N, wl.K).to(torch.bfloat16)        # exact: +-bf16 values
    got = ss1.project(W, p.hash, p.sign, wl.c, wl.BK, wl.BN)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), Wc.view(torch.int16))


def test_project_side_stream_and_no_write_past_end():
    wl = Workload("proj_stream", 9, 99, 0, 768, 128, 2, 64, 64, "bf16")
    vals, bits = make_dense_weight(wl)
    W = to_dev(vals, bits, "bf16")
    p = ss1.DevicePlan.make(wl.plan_seed, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    buf = torch.full((wl.N * wl.Kc + 64,), 12345, dtype=torch.int16, device="cuda")
    out = buf[: wl.N * wl.Kc].view(torch.bfloat16).view(wl.N, wl.Kc)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ss1.project(W, p.hash, p.sign, wl.c, wl.BK, wl.BN, W_c=out, stream=s)
    s.synchronize()
    assert torch.all(buf[wl.N * wl.Kc:] == 12345)
    check(wl, to_host(out), vals.astype(np.float64))
