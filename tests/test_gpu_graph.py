"""The linear layer replayed from a captured HIP graph: every replay equals the eager call bit
for bit, with the program's own eager work and synchronizations between the replays (the path
records only kernel launches: no allocation, copy or fill, when out and workspace are given)."""
import numpy as np
import pytest
import torch

from fp4_block_scaled_amd import synth
from _util import to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mx():
    import fp4_block_scaled_amd as m
    assert torch.cuda.is_available()
    m.lib()
    return m


def _operands(mx, M, K, N, seed):
    a = to_dev_bf16(synth.bits16(synth.to_bf16(synth.normal_f32(seed, (M, K), 1.0))))
    w = to_dev_bf16(synth.bits16(synth.to_bf16(synth.normal_f32(seed + 1, (N, K), 0.02))))
    bias = torch.from_numpy(synth.bits16(synth.to_f16(synth.normal_f32(seed + 2, (N,), 0.01))).view(np.int16)
                            ).view(torch.float16).cuda()
    return a, mx.quantize(w, "mxfp4", layout="tiled"), bias


@pytest.mark.parametrize("M,K,N,calls", [(256, 512, 512, 1), (300, 768, 640, 4), (2048, 1024, 2048, 2)])
def test_linear_graph_replays_equal_eager(mx, M, K, N, calls):
    a, wq, bias = _operands(mx, M, K, N, 52000 + M)
    ws = torch.empty(mx.linear_workspace_bytes(M, K, "mxfp4"), dtype=torch.uint8, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    eager = mx.linear(a, wq, bias)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mx.linear(a, wq, bias, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            mx.linear(a, wq, bias, out=out, workspace=ws)
    other_a, other_w, other_b = _operands(mx, 128, 512, 256, 53000)
    for rep in range(4):
        out.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        # eager work of the program between replays, touching other buffers
        mx.linear(other_a, other_w, other_b)
        torch.cuda.synchronize()
