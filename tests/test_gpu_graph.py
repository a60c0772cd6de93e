"""The forward entry points under HIP graph capture.

Decode-size calls take microseconds, so a serving loop captures them in a
graph.  The library launches kernels only (no allocation, no memset), so a
captured call must replay to the eager result: each replay here follows eager
work that changes the input buffer in place, and every replay is compared
with an eager call on the same contents (bit for bit: same kernel, same
inputs).
"""
import numpy as np
import pytest

import sketched_parameter_sharing_amd as ss1
from ss1_inputs import WORKLOADS, make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ss1.load()


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def replay_matches_eager(call, x, y, replays=3):
    """Capture call() (which reads x and writes y), then replay it after
    changing x in place; each replay must equal an eager call."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm-up outside the capture (kernel attributes, module load)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    x0 = x.clone()
    for r in range(replays):
        # eager work between replays: a different input in the same buffer
        x.copy_(x0 * (1.0 + 0.25 * r) if r else x0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = y.clone()
        call()
        torch.cuda.synchronize()
        assert torch.equal(got, y), f"replay {r} differs from the eager call"


@pytest.mark.parametrize("name,M,algo", [("llama_gateup_m1", 1, "gemv"), ("llama_down_m1", 2, "gemv"),
                                         ("llama_gateup_m16", 16, "smallm"), ("llama_gateup_m16", 16, "decode"),
                                         ("gpt2s_up", 300, "auto"), ("llama_down_m4096", 300, "fold")])
def test_forward_replays(name, M, algo):
    wl = WORKLOADS[name].with_m(M)
    inp = make_inputs(wl)
    p = ss1.DevicePlan.make(wl.plan_seed, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    x, w = bf16_dev(inp.x_bits), bf16_dev(inp.w_bits)
    y = torch.empty((M, wl.N), dtype=torch.bfloat16, device="cuda")
    replay_matches_eager(lambda: p.forward(x, w, y=y, algo=algo), x, y)


@pytest.mark.parametrize("name,M", [("llama_gateup_m1", 1), ("llama_down_m16", 16)])
def test_forward_fp8w_replays(name, M):
    wl = WORKLOADS[name].with_m(M)
    inp = make_inputs(wl)
    p = ss1.DevicePlan.make(wl.plan_seed, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    Q, scale = ss1.quantize_fp8(bf16_dev(inp.w_bits))
    x = bf16_dev(inp.x_bits)
    y = torch.empty((M, wl.N), dtype=torch.bfloat16, device="cuda")
    replay_matches_eager(
        lambda: ss1.forward_fp8w(x, Q, scale, p.hash, p.sign, wl.c, wl.BK, wl.BN, y=y), x, y)


@pytest.mark.parametrize("M", [16, 7])
def test_forward_ws_split_replays(M):
    # the column-split decode: two launches (partial tiles into the workspace,
    # then their in-order sum), captured together
    wl = WORKLOADS["llama_down_m16"].with_m(M)
    kernel, nbytes = ss1.forward_ws_query(M, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    assert kernel == "split"
    inp = make_inputs(wl)
    p = ss1.DevicePlan.make(wl.plan_seed, wl.K, wl.N, wl.c, wl.BK, wl.BN)
    x, w = bf16_dev(inp.x_bits), bf16_dev(inp.w_bits)
    y = torch.empty((M, wl.N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    replay_matches_eager(lambda: ss1.forward_ws(x, w, p.hash, p.sign, wl.c, wl.BK, wl.BN, workspace=ws, y=y), x, y)
