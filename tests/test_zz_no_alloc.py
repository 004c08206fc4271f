"""mx_linear_noalloc: the linear layer with the library's static per-GPU workspace, for callers
that cannot allocate.  Its output must equal mx_linear's (same kernels, so bit for bit) on two
calls in a row, the second with a smaller activation, so that the second call runs on what the
first one left in the shared workspace."""
import numpy as np
import pytest
import torch

from fp4_block_scaled_amd import synth
from _util import activation_bits, f16_bits, to_dev_bf16, to_dev_f16, weight_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mx():
    import fp4_block_scaled_amd as m
    m.lib()
    return m


def _pair(mx, a, wq, bias, **kw):
    y_ref = mx.linear(a, wq, bias, **kw)
    y = mx.linear_noalloc(a, wq, bias, **kw)
    torch.cuda.synchronize()
    return y_ref, y


def _equal(y_ref, y):
    if isinstance(y_ref, torch.Tensor):
        assert y.dtype == y_ref.dtype and y.shape == y_ref.shape
        assert torch.equal(y.view(torch.int16 if y.dtype == torch.bfloat16 else torch.int32),
                           y_ref.view(torch.int16 if y_ref.dtype == torch.bfloat16 else torch.int32))
    else:
        assert torch.equal(y.codes, y_ref.codes) and torch.equal(y.scales, y_ref.scales)


@pytest.mark.parametrize("act,out_dtype", [("mxfp4", torch.bfloat16), ("mxfp4", torch.float32),
                                           ("mxfp8", torch.float32), ("nvfp4", torch.bfloat16)])
def test_noalloc_matches_linear_two_calls_second_smaller(mx, act, out_dtype):
    K, N = 1024, 640
    w_bits = weight_bits(N, K, seed=14100)
    w_bf = to_dev_bf16(w_bits)
    if act == "nvfp4":
        wq = mx.quantize_weight_nvfp4(w_bf)
        kw = dict(act_fmt="nvfp4", act_global_scale=mx.nvfp4_global_scale(40.0))
    else:
        wq = mx.quantize(w_bf, "mxfp4", layout="tiled")
        kw = dict(act_fmt=act)
    bias = to_dev_f16(f16_bits(synth.normal_f32(14200, (N,), 0.01)))
    for i, M in enumerate((1100, 300)):  # the second call is smaller than the first
        a = to_dev_bf16(activation_bits(M, K, seed_base=14300 + i))
        y_ref, y = _pair(mx, a, wq, bias, out_dtype=out_dtype, **kw)
        _equal(y_ref, y)


def test_noalloc_lowrank_and_requant_epilogue(mx):
    K, N, R = 768, 512, 32
    wq = mx.quantize(to_dev_bf16(weight_bits(N, K, seed=14400)), "mxfp4", layout="tiled")
    down = to_dev_bf16(synth.bits16(synth.to_bf16(synth.normal_f32(14500, (R, K), 0.02))))
    up = to_dev_bf16(synth.bits16(synth.to_bf16(synth.normal_f32(14600, (N, R), 0.02))))
    lr = mx.LowRank(down, up)
    for i, M in enumerate((700, 65)):
        a = to_dev_bf16(activation_bits(M, K, seed_base=14700 + i))
        y_ref, y = _pair(mx, a, wq, None, act_fmt="mxfp8", lowrank=lr, out_dtype=torch.float32)
        _equal(y_ref, y)
        h_ref, h = _pair(mx, a, wq, None, epilogue="bias_gelu_quant_mxfp4_tiled")
        _equal(h_ref, h)


def test_noalloc_rejects_oversized_workspace(mx):
    K = 5120
    wq = mx.quantize(torch.zeros((128, K), dtype=torch.bfloat16, device="cuda"), "mxfp4", layout="tiled")
    M = 24576 + 256  # past the static workspace at K = 5120
    assert mx.linear_workspace_bytes(M, K, "mxfp4") > mx.NOALLOC_SCRATCH_BYTES
    a = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    out = torch.full((M, 128), 5.0, dtype=torch.float32, device="cuda")
    with pytest.raises(mx.MxError, match="static scratch"):
        mx.linear_noalloc(a, wq, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 5.0)
    M = 24576  # the largest that fits
    assert mx.linear_workspace_bytes(M, K, "mxfp4") <= mx.NOALLOC_SCRATCH_BYTES
    y = mx.linear_noalloc(a[:M], wq, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.all(y == 0)
