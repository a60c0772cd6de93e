"""GPU test of ss1_mlp_forward_static (the MLP pair with its h workspace in
the library's static device array), through the C ABI: two calls in a row,
the second on fewer rows, each bit-identical to ss1_mlp_forward with an h of
the same rows per chunk (the same kernels run on the same chunks)."""
import numpy as np
import pytest

import sketched_parameter_sharing_amd as ss1
from ss1_inputs import draw, f32_to_bf16_bits

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ss1.load()


def bf16(a):
    return torch.from_numpy(f32_to_bf16_bits(a).view(np.int16)).view(torch.bfloat16).cuda()


def layer(seed, K, N, c, BK, BN):
    p = ss1.DevicePlan.make(seed, K, N, c, BK, BN)
    return (bf16(draw("normal002", seed, (N, K // c))), p.hash, p.sign, c, BK, BN)


@pytest.mark.parametrize("K,N1,c", [(1280, 5120, 4), (768, 3072, 2)])
def test_static_matches_workspace_entry_point(K, N1, c):
    up = layer(0x7a00 + c, K, N1, c, 64, 64)
    down = layer(0x7a10 + c, N1, K, c, 64, 64)
    R = ss1.static_rows(N1, 2)
    for M in (R + 1000, 300):            # two chunks, then one smaller call
        x = bf16(draw("normal", 0x7a20 + M, (M, K)))
        y_static = ss1.mlp_forward_static(x, up, down)
        _, y_ws = ss1.mlp_forward(x, up, down, row_chunk=R)
        torch.cuda.synchronize()
        assert torch.equal(y_static.view(torch.int16), y_ws.view(torch.int16)), f"M={M}"


def test_static_empty_input():
    up = layer(0x7a30, 768, 3072, 2, 64, 64)
    down = layer(0x7a31, 3072, 768, 2, 64, 64)
    x = torch.empty((0, 768), dtype=torch.bfloat16, device="cuda")
    y = ss1.mlp_forward_static(x, up, down)
    assert y.shape == (0, 768)
