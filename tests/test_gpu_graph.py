"""The library's calls replayed from captured HIP graphs: every replay equals the eager call bit
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


def _replays_equal_eager(fn, outs, between):
    """Capture fn (which writes only into the tensors `outs`) in a graph; every one of four
    replays, each after the outputs are cleared and followed by unrelated eager work, must
    reproduce the outputs of an eager call bit for bit."""
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for rep in range(4):
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), f"replay {rep}, output {i}"
        between()
        torch.cuda.synchronize()


def _bf16(seed, shape, sigma):
    return to_dev_bf16(synth.bits16(synth.to_bf16(synth.normal_f32(seed, shape, sigma))))


def test_w4a8_lowrank_graph_replays_equal_eager(mx):
    """W4A8 with the rank-32 branch: the fused MXFP8 quantizer + low-rank projection, then the
    GEMM with its low-rank pass."""
    M, K, N, R = 300, 1024, 384, 32
    a, bias = _bf16(54000, (M, K), 1.0), _operands(mx, 8, K, N, 54001)[2]
    wq = mx.quantize(_bf16(54002, (N, K), 0.02), "mxfp4", layout="tiled")
    lr = mx.LowRank(_bf16(54003, (R, K), 0.02), _bf16(54004, (N, R), 0.02))
    ws = torch.empty(mx.linear_workspace_bytes(M, K, "mxfp8", R), dtype=torch.uint8, device="cuda")
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    other = _operands(mx, 128, 512, 256, 54005)
    _replays_equal_eager(
        lambda: mx.linear(a, wq, bias, act_fmt="mxfp8", lowrank=lr, out_dtype=torch.float32, out=out, workspace=ws),
        [out], lambda: mx.linear(*other))


def test_ffn_pair_graph_replays_equal_eager(mx):
    """The FFN pair: GELU + MXFP4 re-quantization into the tiled layout, then the second linear
    on those codes."""
    M, K, H, N = 300, 512, 1024, 512
    a = _bf16(55000, (M, K), 1.0)
    w0 = mx.quantize(_bf16(55001, (H, K), 0.03), "mxfp4", layout="tiled")
    w2 = mx.quantize(_bf16(55002, (N, H), 0.03), "mxfp4", layout="tiled")
    b0, b2 = _operands(mx, 8, K, H, 55003)[2], _operands(mx, 8, H, N, 55004)[2]
    hq = mx.empty_qmatrix(M, H, "mxfp4", layout="tiled")
    ws = torch.empty(mx.linear_workspace_bytes(M, K, "mxfp4"), dtype=torch.uint8, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def ffn():
        mx.linear(a, w0, b0, epilogue="bias_gelu_quant_mxfp4_tiled", out=hq, workspace=ws)
        mx.linear_q(hq, w2, b2, out=y)
    other = _operands(mx, 128, 512, 256, 55005)
    _replays_equal_eager(ffn, [hq.codes, hq.scales, y], lambda: mx.linear(*other))


def test_norm_quantize_graph_replays_equal_eager(mx):
    """The producer fused with the quantizer (LayerNorm + modulation, tiled MXFP4 output)."""
    M, C = 257, 3072
    x = _bf16(56000, (M, C), 2.0)
    scale = torch.from_numpy(synth.normal_f32(56001, (C,), 0.1)).cuda()
    shift = torch.from_numpy(synth.normal_f32(56002, (C,), 0.1)).cuda()
    q = mx.empty_qmatrix(M, C, "mxfp4", layout="tiled")
    other = _bf16(56003, (64, 1024), 1.0)
    _replays_equal_eager(lambda: mx.norm_quantize(x, scale=scale, shift=shift, out=q),
                         [q.codes, q.scales], lambda: mx.quantize(other, "mxfp4"))


def test_attention_graph_replays_equal_eager(mx):
    """Q/K quantization, V^T quantization and the microscaled attention in one graph."""
    S, H, D = 700, 2, 128
    q, k, v = (_bf16(57000 + i, (S, H * D), 1.0) for i in range(3))
    qg, kg = mx.quantize(q, "mxfp4"), mx.quantize(k, "mxfp4")
    vv = v.view(S, H, D).transpose(0, 1)
    vt = mx.quantize_vt(vv)
    o = torch.empty((S, H * D), dtype=torch.bfloat16, device="cuda")

    def attn():
        mx.quantize(q, "mxfp4", out=qg)
        mx.quantize(k, "mxfp4", out=kg)
        mx.quantize_vt(vv, out=vt)
        mx.attention(qg, kg, vt, H, layout="shd", out=o)
    outs = [qg.codes, qg.scales, kg.codes, kg.scales, vt[0], vt[1], o]
    other = _bf16(57010, (64, 1024), 1.0)
    _replays_equal_eager(attn, outs, lambda: mx.quantize(other, "mxfp4"))
