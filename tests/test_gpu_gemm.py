"""GPU parity of the block-scaled linear layer against the CPU oracle.

Tolerance (from the task's contract): |y_gpu - y_ref| <= 2e-3 * sum_k |a_k w_k| per element,
before the final BF16 rounding (checked on the FP32 output), plus one binary32 rounding of the
result; the BF16 output must be the RNE of the FP32 output.  Exact special cases are compared
bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle as O
from fp4_block_scaled_amd import synth
from _util import (activation_bits, assert_within, bf16_rne_of_f32, dev_bits16, f16_bits,
                   sample_rows, tile_mx, to_dev_bf16, to_dev_f16, unpack_fp4, weight_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mx():
    import fp4_block_scaled_amd as m
    assert torch.cuda.is_available()
    m.lib()
    return m


def _quant_w(mx, w_bits):
    q = mx.quantize(to_dev_bf16(w_bits), "mxfp4")
    return q


def _mx_case(mx, M, K, N, seed=0, bias=True, act="mxfp4", out_dtype=torch.float32, epi="bias",
             w_fmt="mxfp4"):
    a_bits = activation_bits(M, K, seed_base=11000 + seed)
    w_bits = weight_bits(N, K, seed=11100 + seed)
    b_bits = f16_bits(synth.normal_f32(11200 + seed, (N,), 0.01)) if bias else None
    wq = mx.quantize(to_dev_bf16(w_bits), w_fmt)
    y = mx.linear(to_dev_bf16(a_bits), wq, to_dev_f16(b_bits) if bias else None, act_fmt=act,
                  out_dtype=out_dtype, epilogue=epi)
    torch.cuda.synchronize()
    elem = O.E4M3 if act == "mxfp8" else O.E2M1
    w_elem = O.E4M3 if w_fmt == "mxfp8" else O.E2M1
    ac, as_ = O.quantize_mx_bf16(a_bits, elem)
    wc, ws = O.quantize_mx_bf16(w_bits, w_elem)
    assert np.array_equal(wq.codes.cpu().numpy(), wc) and np.array_equal(wq.scales.cpu().numpy(), ws)
    y_ref, abs_sum = O.linear_ref_mx(ac, as_, elem, wc, ws, K, b_bits, w_elem=w_elem)
    return y, y_ref, abs_sum, (a_bits, wq, b_bits)


@pytest.mark.parametrize("M,K,N", [(256, 512, 512), (300, 1024, 640), (1, 256, 256), (37, 288, 96),
                                   (64, 32, 32), (513, 768, 1024), (260, 384, 200), (300, 640, 160),
                                   (700, 1280, 96)])
def test_mxfp4_linear_f32_vs_oracle(mx, M, K, N):
    y, y_ref, abs_sum, _ = _mx_case(mx, M, K, N, seed=M + K + N)
    assert_within(y.cpu().numpy(), y_ref, abs_sum)


@pytest.mark.parametrize("M,K,N", [(300, 1024, 640), (77, 256, 100), (260, 384, 200)])
def test_bf16_output_is_rne_of_f32_output(mx, M, K, N):
    """Both BF16 store paths: staged through LDS (N % 8 == 0) and direct (N = 100)."""
    a_bits = activation_bits(M, K, seed_base=12000)
    wq = _quant_w(mx, weight_bits(N, K, seed=12100))
    b = to_dev_f16(f16_bits(synth.normal_f32(12200, (N,), 0.01)))
    a = to_dev_bf16(a_bits)
    y32 = mx.linear(a, wq, b, out_dtype=torch.float32)
    y16 = mx.linear(a, wq, b, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dev_bits16(y16), bf16_rne_of_f32(y32.cpu().numpy()))


def test_exact_grid_case_is_bit_exact(mx):
    """Grid-valued operands with unit scales: every partial sum is a multiple of 1/4 below 2^24,
    so any fp32 summation order gives the exact result."""
    rng = np.random.default_rng(3)
    M, K, N = 96, 2048, 160
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float32)
    a = rng.choice(grid, size=(M, K)) * rng.choice([-1, 1], size=(M, K))
    w = rng.choice(grid, size=(N, K)) * rng.choice([-1, 1], size=(N, K))
    a[:, ::32] = 6.0  # every block max is 6 -> unit scale
    w[:, ::32] = 4.0
    a_bits = synth.bits16(synth.to_bf16(a.astype(np.float32)))
    w_bits = synth.bits16(synth.to_bf16(w.astype(np.float32)))
    wq = _quant_w(mx, w_bits)
    y = mx.linear(to_dev_bf16(a_bits), wq, None, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = a.astype(np.float64) @ w.astype(np.float64).T
    np.testing.assert_array_equal(y.cpu().numpy().astype(np.float64), ref)


def test_one_hot_weight_and_zero_activation(mx):
    M, K, N = 130, 512, 64
    a_bits = activation_bits(M, K, seed_base=12300)
    w = np.zeros((N, K), dtype=np.float32)
    for n in range(N):
        w[n, 7 * n] = 1.0
    wq = _quant_w(mx, synth.bits16(synth.to_bf16(w)))
    b_bits = f16_bits(synth.normal_f32(12400, (N,), 0.01))
    bias = O.f16_values(b_bits)
    y = mx.linear(to_dev_bf16(a_bits), wq, to_dev_f16(b_bits), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ac, as_ = O.quantize_mx_bf16(a_bits)
    adeq = O.dequantize_mx(ac, as_, K)
    ref = (adeq[:, 0:7 * N:7] + bias).astype(np.float32)  # one fp32 rounding of â + b
    np.testing.assert_array_equal(y.cpu().numpy(), ref)
    y0 = mx.linear(torch.zeros((M, K), dtype=torch.bfloat16, device="cuda"), wq,
                   to_dev_f16(b_bits), out_dtype=torch.float32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y0.cpu().numpy(), np.broadcast_to(bias.astype(np.float32), (M, N)))


def test_linear_deterministic_and_no_writes_past_output(mx):
    M, K, N = 200, 1024, 384
    a = to_dev_bf16(activation_bits(M, K, seed_base=12500))
    wq = _quant_w(mx, weight_bits(N, K, seed=12600))
    buf = torch.full((M * N + 8192,), -7.0, dtype=torch.float32, device="cuda")
    out = buf[: M * N].view(M, N)
    mx.linear(a, wq, None, out_dtype=torch.float32, out=out)
    first = out.clone()
    mx.linear(a, wq, None, out_dtype=torch.float32, out=out)
    torch.cuda.synchronize()
    assert torch.equal(first, out)
    assert torch.all(buf[M * N:] == -7.0)


def test_empty_activation_is_noop(mx):
    wq = _quant_w(mx, weight_bits(64, 256, seed=12700))
    y = mx.linear(torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda"), wq)
    torch.cuda.synchronize()
    assert y.shape == (0, 64)


def test_validation_failure_writes_nothing(mx):
    M, K, N = 64, 256, 64
    a = to_dev_bf16(activation_bits(M, K, seed_base=12800))
    wq = _quant_w(mx, weight_bits(N, K, seed=12900))
    out = torch.full((M, N), 3.0, dtype=torch.float32, device="cuda")
    small_ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(mx.MxError, match="WORKSPACE"):
        mx.linear(a, wq, None, out_dtype=torch.float32, out=out, workspace=small_ws)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)


def test_binding_rejects_bad_out_bias_and_lowrank(mx):
    """linear / linear_q check out (shape, dtype, layout), bias (length, dtype, contiguity) and
    the low-rank factors (dtype, shapes, contiguity) on the host and raise before any launch: the
    sentinel output stays untouched."""
    M, K, N = 64, 256, 128
    a = to_dev_bf16(activation_bits(M, K, seed_base=13000))
    wq = _quant_w(mx, weight_bits(N, K, seed=13100))
    aq = mx.quantize(a, "mxfp4")
    sentinel = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    bias = torch.zeros(N, dtype=torch.float16, device="cuda")
    down = torch.zeros((32, K), dtype=torch.bfloat16, device="cuda")
    up = torch.zeros((N, 32), dtype=torch.bfloat16, device="cuda")
    bad_calls = [
        lambda: mx.linear(a, wq, out=torch.empty((M, N - 8), dtype=torch.float32, device="cuda")),
        lambda: mx.linear(a, wq, out=torch.empty((M + 1, N), dtype=torch.float32, device="cuda")),
        lambda: mx.linear(a, wq, out=torch.empty((M, N), dtype=torch.float16, device="cuda")),
        lambda: mx.linear(a, wq, out=torch.empty((N, M), dtype=torch.float32, device="cuda").t()),
        lambda: mx.linear(a, wq, out=torch.empty((M, N), dtype=torch.float32)),
        lambda: mx.linear(a, wq, bias=torch.zeros(N - 1, dtype=torch.float16, device="cuda"), out=sentinel),
        lambda: mx.linear(a, wq, bias=torch.zeros(N, dtype=torch.float32, device="cuda"), out=sentinel),
        lambda: mx.linear(a, wq, bias=torch.zeros(2 * N, dtype=torch.float16, device="cuda")[::2], out=sentinel),
        lambda: mx.linear(a, wq, lowrank=mx.LowRank(down[:, : K - 32], up), out=sentinel),
        lambda: mx.linear(a, wq, lowrank=mx.LowRank(down, up[: N - 1]), out=sentinel),
        lambda: mx.linear(a, wq, lowrank=mx.LowRank(down, torch.zeros((N, 16), dtype=torch.bfloat16,
                                                                       device="cuda")), out=sentinel),
        lambda: mx.linear(a, wq, lowrank=mx.LowRank(down.float(), up), out=sentinel),
        lambda: mx.linear(a, wq, lowrank=mx.LowRank(down, torch.zeros((32, N), dtype=torch.bfloat16,
                                                                       device="cuda").t()), out=sentinel),
        lambda: mx.linear(a, wq, epilogue="bias_gelu_quant_mxfp4", out=sentinel),
        lambda: mx.linear(a, wq, epilogue="bias_gelu_quant_mxfp4_tiled", out=mx.empty_qmatrix(M, N, "mxfp4")),
        lambda: mx.linear(a, wq, epilogue="bias_gelu_quant_mxfp4", out=mx.empty_qmatrix(M, N // 2, "mxfp4")),
        lambda: mx.linear(a, wq, out_dtype=torch.float16),
        lambda: mx.linear_q(aq, wq, out=torch.empty((M, N // 2), dtype=torch.float32, device="cuda")),
        lambda: mx.linear_q(aq, wq, bias=torch.zeros(N + 1, dtype=torch.float16, device="cuda"), out=sentinel),
    ]
    for i, call in enumerate(bad_calls):
        with pytest.raises(mx.MxError):
            call()
    torch.cuda.synchronize()
    assert torch.all(sentinel == 7.0)
    # the output type follows the tensor passed as out, whatever out_dtype says
    y32 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    mx.linear(a, wq, bias, out=y32)
    y16 = mx.linear(a, wq, bias)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dev_bits16(y16), bf16_rne_of_f32(y32.cpu().numpy()))


@pytest.mark.parametrize("act", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("M,K,N", [(300, 1024, 640), (260, 384, 200), (513, 768, 1024)])
def test_tiled_operands_give_identical_results(mx, M, K, N, act):
    """The tiled layout only moves bytes: every layout pairing gives the same output bits."""
    a = to_dev_bf16(activation_bits(M, K, seed_base=16000 + M))
    w_rm = _quant_w(mx, weight_bits(N, K, seed=16100 + N))
    w_t = mx.relayout(w_rm)
    bias = to_dev_f16(f16_bits(synth.normal_f32(16200, (N,), 0.01)))
    a_rm = mx.quantize(a, act)
    a_t = mx.quantize(a, act, layout="tiled")
    ref = mx.linear_q(a_rm, w_rm, bias, out_dtype=torch.float32)
    for aa, ww in ((a_t, w_t), (a_rm, w_t), (a_t, w_rm)):
        assert torch.equal(mx.linear_q(aa, ww, bias, out_dtype=torch.float32), ref)
    assert torch.equal(mx.linear(a, w_t, bias, act_fmt=act, out_dtype=torch.float32), ref)
    assert torch.equal(mx.linear(a, w_rm, bias, act_fmt=act, out_dtype=torch.float32), ref)


# ---------------------------------------------------------------------------------------------
# W4A8 (MXFP8 activations) and the low-rank branch
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,N", [(130, 512, 256), (300, 3072, 384), (77, 384, 200)])
def test_w4a8_linear_vs_oracle(mx, M, K, N):
    y, y_ref, abs_sum, _ = _mx_case(mx, M, K, N, seed=7 * M, act="mxfp8")
    assert_within(y.cpu().numpy(), y_ref, abs_sum)


def _lowrank_case(mx, M, K, N, R, act, bias, w_fmt="mxfp4"):
    a_bits = activation_bits(M, K, seed_base=13000, factor=25.0)
    w_bits = weight_bits(N, K, seed=13100)
    down = synth.bits16(synth.to_bf16(synth.normal_f32(13200, (K, R), 0.02)))
    up = synth.bits16(synth.to_bf16(synth.normal_f32(13300, (R, N), 0.02)))
    b_bits = f16_bits(synth.normal_f32(13400, (N,), 0.01)) if bias else None
    wq = mx.quantize(to_dev_bf16(w_bits), w_fmt)
    w_elem = O.E4M3 if w_fmt == "mxfp8" else O.E2M1
    lr = mx.LowRank(to_dev_bf16(np.ascontiguousarray(down.T)), to_dev_bf16(np.ascontiguousarray(up.T)))
    y = mx.linear(to_dev_bf16(a_bits), wq, to_dev_f16(b_bits) if bias else None, act_fmt=act,
                  lowrank=lr, out_dtype=torch.float32)
    torch.cuda.synchronize()
    elem = O.E4M3 if act == "mxfp8" else O.E2M1
    ac, as_ = O.quantize_mx_bf16(a_bits, elem)
    wc, ws = O.quantize_mx_bf16(w_bits, w_elem)
    y_ref, abs_sum = O.linear_ref_mx(ac, as_, elem, wc, ws, K, b_bits, w_elem=w_elem)
    u_bits, lr_ref, lr_abs = O.lowrank(a_bits, down, up)
    # u is rounded to BF16 from an fp32 (GPU) or exact (oracle) sum: near a rounding midpoint
    # the two may pick neighbouring BF16 values, a change of up to 2^-8 |u_r| per term.
    u = O.bf16_values(u_bits)
    flip = (2.0 ** -8) * (np.abs(u) @ np.abs(O.bf16_values(up)))
    return y, y_ref + lr_ref, abs_sum, 2e-3 * lr_abs + flip


@pytest.mark.parametrize("act", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("R", [32, 16, 64])
def test_lowrank_branch_vs_oracle(mx, act, R):
    y, y_ref, abs_sum, extra = _lowrank_case(mx, 200, 768, 320, R, act, bias=(R == 32))
    assert_within(y.cpu().numpy(), y_ref, abs_sum, extra, what=f"low-rank {act} R={R}")


@pytest.mark.parametrize("act", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("M,K,N,R", [(150, 288, 192, 32), (97, 352, 100, 16), (70, 160, 64, 48)])
def test_lowrank_branch_k_not_multiple_of_128(mx, act, M, K, N, R):
    """K % 128 != 0: the register-staged GEMM with its low-rank pass, and the low-rank down
    projection's partial last 64-element chunk."""
    y, y_ref, abs_sum, extra = _lowrank_case(mx, M, K, N, R, act, bias=(R != 16))
    assert_within(y.cpu().numpy(), y_ref, abs_sum, extra, what=f"low-rank {act} {M}x{K}x{N} R={R}")


@pytest.mark.parametrize("act,w_fmt,M,K,N,R", [
    ("mxfp4", "mxfp4", 256, 512, 512, 0),    # the one-launch small linear
    ("mxfp4", "mxfp4", 600, 1024, 640, 0),   # quantizer + GEMM
    ("mxfp8", "mxfp4", 300, 1024, 384, 32),  # MXFP8 quantizer fused with the low-rank down projection
    ("mxfp4", "mxfp4", 200, 768, 320, 16),   # quantizer, then the low-rank down projection
    ("mxfp8", "mxfp4", 77, 352, 200, 32),    # K % 128 != 0: row-major operands
    ("nvfp4", "nvfp4", 257, 288, 96, 0),
    ("mxfp8", "mxfp8", 130, 512, 256, 0),
])
def test_strided_activation_equals_contiguous(mx, act, w_fmt, M, K, N, R):
    """An activation view with ld_a = K + 64 whose 64 padding columns hold BF16 NaN gives the same
    F32 output, bit for bit, as its contiguous copy: every kernel on the path (quantizers, the
    one-launch small linear, the fused MXFP8 quantizer + low-rank projection) steps rows by ld_a
    and reads no element past K (a NaN read would turn its group's scale and outputs to NaN)."""
    a_bits = activation_bits(M, K, seed_base=16000 + M, factor=20.0)
    w_bits = weight_bits(N, K, seed=16100)
    b = to_dev_f16(f16_bits(synth.normal_f32(16200, (N,), 0.01)))
    wide = np.full((M, K + 64), 0x7FC0, dtype=np.uint16)
    wide[:, :K] = a_bits
    a_wide = to_dev_bf16(wide)
    a_view, a_cont = a_wide[:, :K], to_dev_bf16(a_bits)
    assert a_view.stride(0) == K + 64
    kw = {}
    if w_fmt == "nvfp4":
        wq = mx.quantize_weight_nvfp4(to_dev_bf16(w_bits))
        kw["act_global_scale"] = O.nv_global_scale(40.0)
    else:
        wq = mx.quantize(to_dev_bf16(w_bits), w_fmt)
    if R:
        down = synth.bits16(synth.to_bf16(synth.normal_f32(16300, (R, K), 0.02)))
        up = synth.bits16(synth.to_bf16(synth.normal_f32(16400, (N, R), 0.02)))
        kw["lowrank"] = mx.LowRank(to_dev_bf16(down), to_dev_bf16(up))
    y_view = mx.linear(a_view, wq, b, act_fmt=act, out_dtype=torch.float32, **kw)
    y_cont = mx.linear(a_cont, wq, b, act_fmt=act, out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    assert torch.isfinite(y_cont).all()
    assert torch.equal(y_view, y_cont)


@pytest.mark.parametrize("pad", [40, 4])  # ld_out % 8 == 0: staged BF16 epilogue; % 8 == 4: direct
@pytest.mark.parametrize("odt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("act,w_fmt,M,K,N,R,epi", [
    ("mxfp4", "mxfp4", 256, 512, 512, 0, "bias"),          # the one-launch small linear
    ("mxfp4", "mxfp4", 600, 1024, 640, 0, "bias_gelu"),    # 256 x 128 ring tiles
    ("mxfp4", "mxfp4", 4096, 512, 4096, 0, "bias"),        # ping-pong 256 x 256 tiles
    ("mxfp8", "mxfp4", 300, 1024, 384, 32, "bias"),
    ("nvfp4", "nvfp4", 257, 288, 96, 0, "bias"),
    ("mxfp8", "mxfp8", 130, 512, 256, 0, "bias_gelu"),
])
def test_strided_output_equals_contiguous(mx, act, w_fmt, M, K, N, R, epi, odt, pad):
    """An output view with ld_out = N + pad receives the same bits as a contiguous output, and
    the pad columns of every row keep their sentinel (no write past N)."""
    a = to_dev_bf16(activation_bits(M, K, seed_base=17000 + M, factor=20.0))
    w_bits = weight_bits(N, K, seed=17100)
    b = to_dev_f16(f16_bits(synth.normal_f32(17200, (N,), 0.01)))
    kw = {"act_fmt": act, "epilogue": epi, "out_dtype": odt}
    if w_fmt == "nvfp4":
        wq = mx.quantize_weight_nvfp4(to_dev_bf16(w_bits))
        kw["act_global_scale"] = O.nv_global_scale(40.0)
    else:
        wq = mx.quantize(to_dev_bf16(w_bits), w_fmt, layout="tiled")
    if R:
        kw["lowrank"] = mx.LowRank(to_dev_bf16(synth.bits16(synth.to_bf16(synth.normal_f32(17300, (R, K), 0.02)))),
                                   to_dev_bf16(synth.bits16(synth.to_bf16(synth.normal_f32(17400, (N, R), 0.02)))))
    y = mx.linear(a, wq, b, **kw)
    wide = torch.full((M, N + pad), -7.5, dtype=odt, device="cuda")
    mx.linear(a, wq, b, out=wide[:, :N], **kw)
    torch.cuda.synchronize()
    assert torch.equal(wide[:, :N], y)
    assert bool((wide[:, N:] == -7.5).all())


# ---------------------------------------------------------------------------------------------
# W8A8 (MXFP8 weights and activations), the MXFP8 reference layer
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,N", [(130, 512, 256), (300, 1024, 640), (77, 384, 200), (1, 128, 128),
                                   (513, 768, 1024), (260, 3072, 96)])
def test_w8a8_linear_vs_oracle(mx, M, K, N):
    y, y_ref, abs_sum, _ = _mx_case(mx, M, K, N, seed=5 * M, act="mxfp8", w_fmt="mxfp8")
    assert_within(y.cpu().numpy(), y_ref, abs_sum, what=f"W8A8 {M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N", [(300, 1024, 640), (260, 384, 200)])
def test_w8a8_tiled_operands_and_bf16_output(mx, M, K, N):
    """Every layout pairing gives the same bits, and the BF16 output is the RNE of the FP32 one
    (both store paths: staged for N % 8 == 0 and direct otherwise)."""
    a = to_dev_bf16(activation_bits(M, K, seed_base=16500 + M))
    w_rm = mx.quantize(to_dev_bf16(weight_bits(N, K, seed=16600 + N)), "mxfp8")
    w_t = mx.relayout(w_rm)
    bias = to_dev_f16(f16_bits(synth.normal_f32(16700, (N,), 0.01)))
    a_rm = mx.quantize(a, "mxfp8")
    a_t = mx.quantize(a, "mxfp8", layout="tiled")
    ref = mx.linear_q(a_rm, w_rm, bias, out_dtype=torch.float32)
    for aa, ww in ((a_t, w_t), (a_rm, w_t), (a_t, w_rm)):
        assert torch.equal(mx.linear_q(aa, ww, bias, out_dtype=torch.float32), ref)
    assert torch.equal(mx.linear(a, w_t, bias, act_fmt="mxfp8", out_dtype=torch.float32), ref)
    y16 = mx.linear(a, w_t, bias, act_fmt="mxfp8", out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dev_bits16(y16), bf16_rne_of_f32(ref.cpu().numpy()))


def test_w8a8_lowrank_and_gelu_epilogue(mx):
    y, y_ref, abs_sum, extra = _lowrank_case(mx, 200, 768, 320, 32, "mxfp8", bias=True, w_fmt="mxfp8")
    assert_within(y.cpu().numpy(), y_ref, abs_sum, extra, what="W8A8 low-rank")
    M, K, N = 300, 1024, 640
    a_bits, w_bits, b_bits = _ffn_inputs(M, K, N)
    wq = mx.quantize(to_dev_bf16(w_bits), "mxfp8")
    h = mx.linear(to_dev_bf16(a_bits), wq, to_dev_f16(b_bits), act_fmt="mxfp8", epilogue="bias_gelu",
                  out_dtype=torch.float32)
    torch.cuda.synchronize()
    ac, as_ = O.quantize_mx_bf16(a_bits, O.E4M3)
    wc, ws = O.quantize_mx_bf16(w_bits, O.E4M3)
    y_ref, abs_sum = O.linear_ref_mx(ac, as_, O.E4M3, wc, ws, K, b_bits, w_elem=O.E4M3)
    h_ref = O.gelu_tanh(y_ref)
    tol_y = 2e-3 * abs_sum + 2.0 ** -23 * np.abs(y_ref)
    err = np.abs(h.cpu().numpy().astype(np.float64) - h_ref)
    assert np.all(err <= 1.13 * tol_y + 4e-6 * np.abs(h_ref) + 1e-7)


@pytest.mark.parametrize("M,K,N,R", [(96, 512, 256, 32), (97, 640, 128, 16), (300, 1024, 384, 64),
                                     (33, 384, 256, 48)])
def test_lowrank_zero_down_is_plain_w4a8(mx, M, K, N, R):
    """With L_down = 0 the branch adds exact zeros, so the output equals plain W4A8 bit for bit:
    this also checks that the pass quantizing the activation together with the low-rank input
    (K % 128 == 0) writes the same codes as the standalone quantizer."""
    a = to_dev_bf16(activation_bits(M, K, seed_base=13500))
    wq = _quant_w(mx, weight_bits(N, K, seed=13600))
    lr = mx.LowRank(torch.zeros((R, K), dtype=torch.bfloat16, device="cuda"),
                    to_dev_bf16(synth.bits16(synth.to_bf16(synth.normal_f32(13700, (N, R), 0.02)))))
    y1 = mx.linear(a, wq, None, act_fmt="mxfp8", lowrank=lr, out_dtype=torch.float32)
    y0 = mx.linear(a, wq, None, act_fmt="mxfp8", out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y1, y0)


# ---------------------------------------------------------------------------------------------
# FFN epilogues: GELU and GELU + MXFP4 re-quantization, then the second linear on the codes
# ---------------------------------------------------------------------------------------------
def _ffn_inputs(M, K, N):
    a_bits = activation_bits(M, K, seed_base=14000, factor=30.0)
    w_bits = weight_bits(N, K, seed=14100, sigma=0.01)
    b_bits = f16_bits(synth.normal_f32(14200, (N,), 0.01))
    return a_bits, w_bits, b_bits


def test_gelu_epilogue_vs_oracle(mx):
    M, K, N = 300, 1024, 640
    a_bits, w_bits, b_bits = _ffn_inputs(M, K, N)
    wq = _quant_w(mx, w_bits)
    h = mx.linear(to_dev_bf16(a_bits), wq, to_dev_f16(b_bits), epilogue="bias_gelu",
                  out_dtype=torch.float32)
    torch.cuda.synchronize()
    ac, as_ = O.quantize_mx_bf16(a_bits)
    wc, ws = O.quantize_mx_bf16(w_bits)
    y_ref, abs_sum = O.linear_ref_mx(ac, as_, O.E2M1, wc, ws, K, b_bits)
    h_ref = O.gelu_tanh(y_ref)
    # |gelu'| <= 1.13: the GEMM tolerance propagates scaled by 1.13; plus fp32 tanh error
    tol_y = 2e-3 * abs_sum + 2.0 ** -23 * np.abs(y_ref)
    err = np.abs(h.cpu().numpy().astype(np.float64) - h_ref)
    assert np.all(err <= 1.13 * tol_y + 4e-6 * np.abs(h_ref) + 1e-7)


def test_gelu_requant_epilogue_self_consistent_and_close_to_oracle(mx):
    M, K, N = 300, 1024, 640
    a_bits, w_bits, b_bits = _ffn_inputs(M, K, N)
    wq = _quant_w(mx, w_bits)
    a, b = to_dev_bf16(a_bits), to_dev_f16(b_bits)
    hq = mx.linear(a, wq, b, epilogue="bias_gelu_quant_mxfp4")
    h32 = mx.linear(a, wq, b, epilogue="bias_gelu", out_dtype=torch.float32)
    torch.cuda.synchronize()
    # the codes are exactly Q_MX of the GPU's own fp32 h (same kernel, same accumulation order)
    c_self, s_self = O.quantize_mx_f32(h32.cpu().numpy())
    np.testing.assert_array_equal(hq.scales.cpu().numpy(), s_self)
    np.testing.assert_array_equal(hq.codes.cpu().numpy(), c_self)
    # against the oracle's h: codes may flip only where h sits near a rounding midpoint
    ac, as_ = O.quantize_mx_bf16(a_bits)
    wc, ws = O.quantize_mx_bf16(w_bits)
    y_ref, _ = O.linear_ref_mx(ac, as_, O.E2M1, wc, ws, K, b_bits)
    c_ref, s_ref = O.quantize_mx_f64(O.gelu_tanh(y_ref))
    mism = np.mean(unpack_fp4(c_ref, N) != unpack_fp4(hq.codes.cpu().numpy(), N))
    print(f"re-quantized H code mismatch rate vs oracle: {mism:.2e}")
    assert mism < 1e-2


def test_ffn_pair_second_linear_on_gpu_codes(mx):
    M, K, N = 300, 512, 1024
    a_bits, w_bits, b_bits = _ffn_inputs(M, K, N)
    w2_bits = weight_bits(K, N, seed=14300, sigma=0.01)
    b2_bits = f16_bits(synth.normal_f32(14400, (K,), 0.01))
    wq = _quant_w(mx, w_bits)
    w2q = _quant_w(mx, w2_bits)
    hq = mx.linear(to_dev_bf16(a_bits), wq, to_dev_f16(b_bits), epilogue="bias_gelu_quant_mxfp4")
    y = mx.linear_q(hq, w2q, to_dev_f16(b2_bits), out_dtype=torch.float32)
    torch.cuda.synchronize()
    y_ref, abs_sum = O.linear_ref_mx(hq.codes.cpu().numpy(), hq.scales.cpu().numpy(), O.E2M1,
                                     w2q.codes.cpu().numpy(), w2q.scales.cpu().numpy(), N, b2_bits)
    assert_within(y.cpu().numpy(), y_ref, abs_sum, what="FFN2 on GPU H codes")


def test_tiled_requant_output_feeds_the_next_linear(mx):
    """The tiled re-quantizing epilogue writes exactly the row-major epilogue's codes and scales,
    regrouped (padding rows zero), and FFN2 on them gives the same output bits."""
    M, K, N = 300, 512, 1024
    a_bits, w_bits, b_bits = _ffn_inputs(M, K, N)
    w2_bits = weight_bits(K, N, seed=14300, sigma=0.01)
    b2 = to_dev_f16(f16_bits(synth.normal_f32(14400, (K,), 0.01)))
    a, b = to_dev_bf16(a_bits), to_dev_f16(b_bits)
    wq = mx.relayout(_quant_w(mx, w_bits))
    w2q = mx.relayout(_quant_w(mx, w2_bits))
    h_rm = mx.linear(a, wq, b, epilogue="bias_gelu_quant_mxfp4")
    h_t = mx.linear(a, wq, b, epilogue="bias_gelu_quant_mxfp4_tiled")
    torch.cuda.synchronize()
    assert h_t.layout == mx.TILED
    tc, ts = tile_mx(h_rm.codes.cpu().numpy(), h_rm.scales.cpu().numpy(), M, N, fp8=False)
    np.testing.assert_array_equal(h_t.codes.cpu().numpy(), tc)
    np.testing.assert_array_equal(h_t.scales.cpu().numpy(), ts)
    y_rm = mx.linear_q(h_rm, w2q, b2, out_dtype=torch.float32)
    y_t = mx.linear_q(h_t, w2q, b2, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y_rm, y_t)


# ---------------------------------------------------------------------------------------------
# NVFP4
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,N", [(300, 1024, 640), (64, 512, 256), (257, 288, 96)])
def test_nvfp4_linear_vs_oracle(mx, M, K, N):
    a_bits = activation_bits(M, K, seed_base=15000, factor=30.0)
    w_bits = weight_bits(N, K, seed=15100, sigma=0.01)
    b_bits = f16_bits(synth.normal_f32(15200, (N,), 0.01))
    sg_a = O.nv_global_scale(40.0)
    wq = mx.quantize_weight_nvfp4(to_dev_bf16(w_bits))
    sg_w = wq.global_scale
    assert sg_w == O.nv_global_scale(O.absmax_bf16(w_bits))
    y = mx.linear(to_dev_bf16(a_bits), wq, to_dev_f16(b_bits), act_fmt="nvfp4",
                  act_global_scale=sg_a, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ac, as_ = O.quantize_nv_bf16(a_bits, sg_a)
    wc, ws = O.quantize_nv_bf16(w_bits, sg_w)
    assert np.array_equal(wq.codes.cpu().numpy(), wc) and np.array_equal(wq.scales.cpu().numpy(), ws)
    y_ref, abs_sum = O.linear_ref_nv(ac, as_, sg_a, wc, ws, sg_w, K, b_bits)
    assert_within(y.cpu().numpy(), y_ref, abs_sum, what="NVFP4 linear")


def test_activation_past_2_31_elements(mx):
    """An activation of 262181 x 8192 BF16 values (2.15e9 elements, 4.3 GB: past 2^31 elements and
    2^32 bytes; seeded on the device, the sampled rows copied back for the oracle).  The row-major
    MXFP4, MXFP8 and NVFP4 quantizers' codes and scales, and the F32 output of the linear (tiled
    quantizer, ping-pong GEMM), are checked against the oracle on rows at the start, on both sides
    of element 2^31 (row 262144 starts at byte 2^32) and at the end; the absolute maximum against
    torch's."""
    M, K, N = 262181, 8192, 256
    assert M * K > 2 ** 31 and 262144 * K == 2 ** 31
    g = torch.Generator(device="cuda").manual_seed(18000)
    a = torch.randn((M, K), generator=g, device="cuda", dtype=torch.bfloat16)
    rows = np.array([0, 1, 2, 262142, 262143, 262144, 262145, 262150, M - 2, M - 1])
    idx = torch.from_numpy(rows).cuda()
    a_rows = synth.bits16(a[idx].cpu())
    w_bits = weight_bits(N, K, seed=18100)
    b_bits = f16_bits(synth.normal_f32(18200, (N,), 0.01))
    wq = mx.quantize(to_dev_bf16(w_bits), "mxfp4", layout="tiled")
    q = mx.quantize(a, "mxfp4")
    y = mx.linear(a, wq, to_dev_f16(b_bits), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ac, as_ = O.quantize_mx_bf16(a_rows)
    np.testing.assert_array_equal(q.codes[idx].cpu().numpy(), ac)
    np.testing.assert_array_equal(q.scales[idx].cpu().numpy(), as_)
    wc, ws = O.quantize_mx_bf16(w_bits)
    y_ref, abs_sum = O.linear_ref_mx(ac, as_, O.E2M1, wc, ws, K, b_bits)
    assert_within(y[idx].cpu().numpy(), y_ref, abs_sum, what="activation past 2^31 elements")
    del q, y
    # the MXFP8 and NVFP4 quantizers and the absolute maximum on the same activation
    q8 = mx.quantize(a, "mxfp8")
    c8, s8 = O.quantize_mx_bf16(a_rows, O.E4M3)
    np.testing.assert_array_equal(q8.codes[idx].cpu().numpy(), c8)
    np.testing.assert_array_equal(q8.scales[idx].cpu().numpy(), s8)
    del q8
    sg = O.nv_global_scale(40.0)
    qn = mx.quantize(a, "nvfp4", global_scale=sg)
    cn, sn = O.quantize_nv_bf16(a_rows, sg)
    np.testing.assert_array_equal(qn.codes[idx].cpu().numpy(), cn)
    np.testing.assert_array_equal(qn.scales[idx].cpu().numpy(), sn)
    del qn
    assert float(mx.absmax(a)) == float(a.abs().max().float())


@pytest.mark.parametrize("odt", [torch.bfloat16, torch.float32])
def test_output_past_2_31_elements(mx, odt):
    """A 262181 x 8192 output (2.15e9 elements; row 262144 starts at element 2^31) from K = 256:
    the BF16 output (staged epilogue) and the F32 output (direct epilogue, 8.6 GB) against the
    oracle on rows at the start, on both sides of the boundary and at the end."""
    M, K, N = 262181, 256, 8192
    assert M * N > 2 ** 31 and 262144 * N == 2 ** 31
    g = torch.Generator(device="cuda").manual_seed(18300)
    a = torch.randn((M, K), generator=g, device="cuda", dtype=torch.bfloat16)
    rows = np.array([0, 1, 262142, 262143, 262144, 262145, M - 2, M - 1])
    idx = torch.from_numpy(rows).cuda()
    a_rows = synth.bits16(a[idx].cpu())
    w_bits = weight_bits(N, K, seed=18400)
    b_bits = f16_bits(synth.normal_f32(18500, (N,), 0.01))
    wq = mx.quantize(to_dev_bf16(w_bits), "mxfp4", layout="tiled")
    y = mx.linear(a, wq, to_dev_f16(b_bits), out_dtype=odt)
    torch.cuda.synchronize()
    got = y[idx].float().cpu().numpy()
    del y
    ac, as_ = O.quantize_mx_bf16(a_rows)
    wc, ws = O.quantize_mx_bf16(w_bits)
    y_ref, abs_sum = O.linear_ref_mx(ac, as_, O.E2M1, wc, ws, K, b_bits)
    if odt == torch.float32:
        assert_within(got, y_ref, abs_sum, what="output past 2^31 elements")
    else:  # BF16: one rounding of a value within the tolerance
        assert np.all(np.abs(got - y_ref) <= 2e-3 * abs_sum + 2.0 ** -8 * np.abs(y_ref) + 1e-30)


@pytest.mark.parametrize("epi", ["bias", "bias_gelu", "bias_gelu_quant_mxfp4", "bias_gelu_quant_mxfp4_tiled"])
def test_pingpong_tile_ragged(mx, epi):
    """A grid of 17 x 17 256 x 256 tiles (at least one per compute unit) takes the ping-pong
    W4A4 kernel: ragged M and N, 6 K chunks, every epilogue, against the oracle on sampled rows
    (the BF16 output as the RNE of the F32 one; the re-quantized codes as Q_MX of the GPU's own
    GELU output)."""
    M, K, N = 4177, 768, 4224  # N % 128 == 0 (tiled re-quantized output), N % 256 != 0
    assert ((M + 255) // 256) * ((N + 255) // 256) >= 256
    a_bits = activation_bits(M, K, seed_base=17000)
    w_bits = weight_bits(N, K, seed=17100)
    b_bits = f16_bits(synth.normal_f32(17200, (N,), 0.01))
    a, bias = to_dev_bf16(a_bits), to_dev_f16(b_bits)
    wq = mx.quantize(to_dev_bf16(w_bits), "mxfp4", layout="tiled")
    rows = sample_rows(M, 400)
    idx = torch.from_numpy(rows).cuda()
    ac, as_ = O.quantize_mx_bf16(a_bits[rows])
    wc, ws = O.quantize_mx_bf16(w_bits)
    y_ref, abs_sum = O.linear_ref_mx(ac, as_, O.E2M1, wc, ws, K, b_bits)
    if epi in ("bias", "bias_gelu"):
        y32 = mx.linear(a, wq, bias, epilogue=epi, out_dtype=torch.float32)
        y16 = mx.linear(a, wq, bias, epilogue=epi)
        torch.cuda.synchronize()
        ys = y32[idx].cpu().numpy()
        np.testing.assert_array_equal(dev_bits16(y16[idx]), bf16_rne_of_f32(ys))
        if epi == "bias":
            assert_within(ys, y_ref, abs_sum, what="ping-pong tile")
        else:
            tol = 2e-3 * abs_sum + 2.0 ** -23 * np.abs(y_ref)
            h_ref = O.gelu_tanh(y_ref)
            assert np.all(np.abs(ys - h_ref) <= 1.13 * tol + 4e-6 * np.abs(h_ref) + 1e-7)
    else:
        h32 = mx.linear(a, wq, bias, epilogue="bias_gelu", out_dtype=torch.float32)
        hq = mx.linear(a, wq, bias, epilogue=epi)
        if epi.endswith("tiled"):
            hq = mx.relayout(hq)
        torch.cuda.synchronize()
        c_self, s_self = O.quantize_mx_f32(h32[idx].cpu().numpy())
        np.testing.assert_array_equal(hq.scales[idx].cpu().numpy(), s_self)
        np.testing.assert_array_equal(hq.codes[idx].cpu().numpy(), c_self)


# ---------------------------------------------------------------------------------------------
# full workload sizes, in the launch configuration the benchmark times (sampled rows)
# ---------------------------------------------------------------------------------------------
FULL_SAMPLE = 1024  # seeded rows per full-size case, plus the first 32 and the last 96 (the M-tail)


def _full_mx(mx, wl_name, act, nsample=FULL_SAMPLE, w_fmt="mxfp4"):
    wl = synth.WORKLOADS[wl_name]
    a_bits = synth.bits16(synth.to_bf16(wl.activation()))
    w_bits = synth.bits16(synth.to_bf16(wl.weight()))
    b = wl.bias()
    b_bits = f16_bits(b) if b is not None else None
    wq = mx.relayout(mx.quantize(to_dev_bf16(w_bits), w_fmt))  # the benchmark's prepared (tiled) weight
    a = to_dev_bf16(a_bits)
    rows = sample_rows(wl.M, nsample)
    bias = to_dev_f16(b_bits) if b is not None else None
    y = mx.linear(a, wq, bias, act_fmt=act, out_dtype=torch.float32)
    y16 = mx.linear(a, wq, bias, act_fmt=act, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    idx = torch.from_numpy(rows).cuda()
    ys = y[idx].cpu().numpy()
    np.testing.assert_array_equal(dev_bits16(y16[idx]), bf16_rne_of_f32(ys))
    del y, y16
    elem = O.E4M3 if act == "mxfp8" else O.E2M1
    w_elem = O.E4M3 if w_fmt == "mxfp8" else O.E2M1
    ac, as_ = O.quantize_mx_bf16(a_bits[rows], elem)
    wc, ws = O.quantize_mx_bf16(w_bits, w_elem)
    y_ref, abs_sum = O.linear_ref_mx(ac, as_, elem, wc, ws, wl.K, b_bits, w_elem=w_elem)
    return assert_within(ys, y_ref, abs_sum, what=wl_name)


def test_full_size_wan_a14b_attention_projection(mx):
    r = _full_mx(mx, "wan_a14b_attn_75600x5120x5120", "mxfp4")
    print(f"max err/tol {r:.3f}")


def test_full_size_w4a8(mx):
    _full_mx(mx, "wan_ti2v5b_w4a8_4290x3072x14336", "mxfp8")


def test_full_size_w8a8(mx):
    r = _full_mx(mx, "wan_a14b_w8a8_75600x5120x5120", "mxfp8", w_fmt="mxfp8")
    print(f"max err/tol {r:.3f}")


@pytest.mark.parametrize("name", ["wan_ti2v5b_w4a8_4290x3072x3072", "wan_ti2v5b_w4a8_4290x3072x14336"])
def test_full_size_w4a8_with_lowrank_branch(mx, name):
    """The W4A8 SVDQuant workloads as the benchmark runs them (N = 3072 and 14336): MXFP8
    activations, prepared MXFP4 weight, rank-32 low-rank branch (no bias), sampled rows against
    the oracle."""
    wl = synth.WORKLOADS[name]
    a_bits = synth.bits16(synth.to_bf16(wl.activation()))
    w_bits = synth.bits16(synth.to_bf16(wl.weight()))
    down = synth.bits16(synth.to_bf16(wl.lora_down()))
    up = synth.bits16(synth.to_bf16(wl.lora_up()))
    wq = mx.relayout(_quant_w(mx, w_bits))
    lr = mx.LowRank(to_dev_bf16(np.ascontiguousarray(down.T)), to_dev_bf16(np.ascontiguousarray(up.T)))
    y = mx.linear(to_dev_bf16(a_bits), wq, None, act_fmt="mxfp8", lowrank=lr, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = sample_rows(wl.M, FULL_SAMPLE)
    ys = y[torch.from_numpy(rows).cuda()].cpu().numpy()
    ac, as_ = O.quantize_mx_bf16(a_bits[rows], O.E4M3)
    wc, ws = O.quantize_mx_bf16(w_bits)
    y_ref, abs_sum = O.linear_ref_mx(ac, as_, O.E4M3, wc, ws, wl.K, None)
    u_bits, lr_ref, lr_abs = O.lowrank(np.ascontiguousarray(a_bits[rows]), down, up)
    flip = (2.0 ** -8) * (np.abs(O.bf16_values(u_bits)) @ np.abs(O.bf16_values(up)))
    assert_within(ys, y_ref + lr_ref, abs_sum, 2e-3 * lr_abs + flip, what=f"W4A8 + low-rank, {name}")


def test_full_size_w4a4_with_lowrank_branch(mx):
    """W4A4 SVDQuant (MXFP4 activations + rank-32 BF16 branch, the W4A8 page's experimental
    activation format) at the A14B attention-projection shape 75600 x 5120 x 5120, factors
    N(0, 0.02) from the workload's seed space, FP16 bias; sampled rows against the oracle."""
    wl = synth.WORKLOADS["wan_a14b_attn_75600x5120x5120"]
    R = 32
    a_bits = synth.bits16(synth.to_bf16(wl.activation()))
    w_bits = synth.bits16(synth.to_bf16(wl.weight()))
    b_bits = f16_bits(wl.bias())
    down = synth.bits16(synth.to_bf16(synth.normal_f32(wl.seed_base + synth.T_LDOWN, (wl.K, R), 0.02)))
    up = synth.bits16(synth.to_bf16(synth.normal_f32(wl.seed_base + synth.T_LUP, (R, wl.N), 0.02)))
    wq = mx.relayout(_quant_w(mx, w_bits))
    lr = mx.LowRank(to_dev_bf16(np.ascontiguousarray(down.T)), to_dev_bf16(np.ascontiguousarray(up.T)))
    y = mx.linear(to_dev_bf16(a_bits), wq, to_dev_f16(b_bits), lowrank=lr, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = sample_rows(wl.M, FULL_SAMPLE)
    ys = y[torch.from_numpy(rows).cuda()].cpu().numpy()
    del y
    ac, as_ = O.quantize_mx_bf16(a_bits[rows])
    wc, ws = O.quantize_mx_bf16(w_bits)
    y_ref, abs_sum = O.linear_ref_mx(ac, as_, O.E2M1, wc, ws, wl.K, b_bits)
    u_bits, lr_ref, lr_abs = O.lowrank(np.ascontiguousarray(a_bits[rows]), down, up)
    flip = (2.0 ** -8) * (np.abs(O.bf16_values(u_bits)) @ np.abs(O.bf16_values(up)))
    assert_within(ys, y_ref + lr_ref, abs_sum, 2e-3 * lr_abs + flip, what="W4A4 + low-rank, full size")


def test_full_size_ffn_pair(mx):
    """The FFN pair at 75600 x 5120 -> 13824 -> 5120 as the benchmark runs it (FFN0 writes H
    tiled, FFN2 reads it), on sampled rows: FFN0's fp32 h against the oracle, the H codes
    against Q_MX of the GPU's own h, and FFN2 against the oracle on the GPU's H codes."""
    wl = synth.WORKLOADS["wan_a14b_ffn_75600x5120x13824"]
    a_bits = synth.bits16(synth.to_bf16(wl.activation()))
    w_bits = synth.bits16(synth.to_bf16(wl.weight()))
    w2_bits = synth.bits16(synth.to_bf16(wl.weight2()))
    b_bits, b2_bits = f16_bits(wl.bias()), f16_bits(wl.bias2())
    a = to_dev_bf16(a_bits)
    wq, w2q = mx.relayout(_quant_w(mx, w_bits)), mx.relayout(_quant_w(mx, w2_bits))
    rows = sample_rows(wl.M, FULL_SAMPLE)
    idx = torch.from_numpy(rows).cuda()
    h32 = mx.linear(a, wq, to_dev_f16(b_bits), epilogue="bias_gelu", out_dtype=torch.float32)
    torch.cuda.synchronize()
    h32s = h32[idx].cpu().numpy()
    del h32
    hq = mx.linear(a, wq, to_dev_f16(b_bits), epilogue="bias_gelu_quant_mxfp4_tiled")
    y = mx.linear_q(hq, w2q, to_dev_f16(b2_bits), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ys = y[idx].cpu().numpy()
    del y
    h_rm = mx.relayout(hq)
    torch.cuda.synchronize()
    hc, hs = h_rm.codes[idx].cpu().numpy(), h_rm.scales[idx].cpu().numpy()
    # FFN0 h against the oracle (GELU-propagated GEMM tolerance, as in the small-shape test)
    ac, as_ = O.quantize_mx_bf16(a_bits[rows])
    wc, ws = O.quantize_mx_bf16(w_bits)
    y0_ref, abs0 = O.linear_ref_mx(ac, as_, O.E2M1, wc, ws, wl.K, b_bits)
    h_ref = O.gelu_tanh(y0_ref)
    err = np.abs(h32s.astype(np.float64) - h_ref)
    tol_y = 2e-3 * abs0 + 2.0 ** -23 * np.abs(y0_ref)
    assert np.all(err <= 1.13 * tol_y + 4e-6 * np.abs(h_ref) + 1e-7)
    # H codes are exactly Q_MX of the GPU's own h
    c_self, s_self = O.quantize_mx_f32(h32s)
    np.testing.assert_array_equal(hs, s_self)
    np.testing.assert_array_equal(hc, c_self)
    # FFN2 on the GPU's H codes
    w2c, w2s = O.quantize_mx_bf16(w2_bits)
    y_ref, abs2 = O.linear_ref_mx(hc, hs, O.E2M1, w2c, w2s, wl.N, b2_bits)
    assert_within(ys, y_ref, abs2, what="FFN2, full size")


def test_full_size_nvfp4(mx):
    """The NVFP4 workload (static activation global scale from amax 40, weight global scale from
    its absmax), sampled rows against the oracle."""
    wl = synth.WORKLOADS["wan_a14b_nvfp4_75600x5120x13824"]
    a_bits = synth.bits16(synth.to_bf16(wl.activation()))
    w_bits = synth.bits16(synth.to_bf16(wl.weight()))
    b_bits = f16_bits(wl.bias())
    wq = mx.quantize_weight_nvfp4(to_dev_bf16(w_bits))
    sg_a = mx.nvfp4_global_scale(wl.act_amax_static)
    y = mx.linear(to_dev_bf16(a_bits), wq, to_dev_f16(b_bits), act_fmt="nvfp4",
                  act_global_scale=sg_a, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = sample_rows(wl.M, FULL_SAMPLE)
    ys = y[torch.from_numpy(rows).cuda()].cpu().numpy()
    del y
    assert sg_a == O.nv_global_scale(wl.act_amax_static)
    sg_w = O.nv_global_scale(float(np.max(np.abs(O.bf16_values(w_bits)))))
    assert wq.global_scale == sg_w
    ac, as_ = O.quantize_nv_bf16(a_bits[rows], sg_a)
    wc, ws = O.quantize_nv_bf16(w_bits, sg_w)
    y_ref, abs_sum = O.linear_ref_nv(ac, as_, sg_a, wc, ws, sg_w, wl.K, b_bits)
    assert_within(ys, y_ref, abs_sum, what="NVFP4, full size")


@pytest.mark.parametrize("act,M,K,N", [(a, 300, 512, 256) for a in ("mxfp4", "mxfp8", "nvfp4")] +
                         [(a, 600, 1024, 512) for a in ("mxfp4", "mxfp8", "nvfp4")] +
                         [("mxfp4", 4096, 256, 4096)])  # 256 tiles of 256 x 256: the ping-pong kernel
def test_nan_and_inf_activations_make_their_rows_nan(mx, act, M, K, N):
    """A NaN or an infinity in an activation block quantizes to the NaN scale (0xFF for E8M0,
    0x7F for E4M3) with zero codes; the block then decodes to NaN, so every output of that row is
    NaN, in the oracle's dequantize-then-GEMM and on the GPU.  The other rows are unaffected."""
    a_bits = activation_bits(M, K, seed_base=16000 + M, factor=30.0)
    a_bits[3, 40] = 0x7FC0     # NaN
    a_bits[100, K - 1] = 0x7F80  # +Inf
    a_bits[M - 1, 0] = 0xFF80    # -Inf, in the last row
    bad = np.zeros(M, dtype=bool)
    bad[[3, 100, M - 1]] = True
    w_bits = weight_bits(N, K, seed=16100, sigma=0.02)
    b_bits = f16_bits(synth.normal_f32(16200, (N,), 0.01))
    if act == "nvfp4":
        sg_a = O.nv_global_scale(40.0)
        wq = mx.quantize_weight_nvfp4(to_dev_bf16(w_bits))
        y = mx.linear(to_dev_bf16(a_bits), wq, to_dev_f16(b_bits), act_fmt="nvfp4",
                      act_global_scale=sg_a, out_dtype=torch.float32)
        ac, as_ = O.quantize_nv_bf16(a_bits, sg_a)
        wc, ws = O.quantize_nv_bf16(w_bits, wq.global_scale)
        y_ref, abs_sum = O.linear_ref_nv(ac, as_, sg_a, wc, ws, wq.global_scale, K, b_bits)
    else:
        wq = mx.quantize(to_dev_bf16(w_bits), "mxfp4")
        y = mx.linear(to_dev_bf16(a_bits), wq, to_dev_f16(b_bits), act_fmt=act, out_dtype=torch.float32)
        elem = O.E4M3 if act == "mxfp8" else O.E2M1
        ac, as_ = O.quantize_mx_bf16(a_bits, elem)
        wc, ws = O.quantize_mx_bf16(w_bits, O.E2M1)
        y_ref, abs_sum = O.linear_ref_mx(ac, as_, elem, wc, ws, K, b_bits)
    torch.cuda.synchronize()
    yg = y.cpu().numpy()
    assert np.isnan(y_ref[bad]).all() and np.isfinite(y_ref[~bad]).all()
    assert np.isnan(yg[bad]).all(), f"{act}: rows with a NaN scale are not all NaN on the GPU"
    assert_within(yg[~bad], y_ref[~bad], abs_sum[~bad], what=f"{act} linear, finite rows")


@pytest.mark.parametrize("M,K,N", [(256, 512, 512), (1, 128, 64), (77, 384, 200), (300, 896, 96),
                                   (512, 256, 512), (2048, 128, 128), (130, 640, 1024)])
@pytest.mark.parametrize("layout", ["row_major", "tiled"])
def test_small_linear_one_launch_equals_quantizer_plus_gemm(mx, M, K, N, layout):
    """Small W4A4 grids run quantization and GEMM in one launch; its output bits equal those of
    the quantizer followed by the GEMM on the same codes (same MFMA pairing and order), for the
    bias and GELU epilogues, BF16 and F32 outputs, with and without bias, ragged M and N."""
    a = to_dev_bf16(activation_bits(M, K, seed_base=17000 + M + K))
    w = mx.quantize(to_dev_bf16(weight_bits(N, K, seed=17100 + N)), "mxfp4")
    if layout == "tiled":
        w = mx.relayout(w)
    bias = to_dev_f16(f16_bits(synth.normal_f32(17200 + N, (N,), 0.01)))
    aq = mx.quantize(a, "mxfp4")
    for b in (bias, None):
        for epi in ("bias", "bias_gelu"):
            for od in (torch.float32, torch.bfloat16):
                one = mx.linear(a, w, b, epilogue=epi, out_dtype=od)
                two = mx.linear_q(aq, w, b, epilogue=epi, out_dtype=od)
                torch.cuda.synchronize()
                assert torch.equal(one.view(torch.int16), two.view(torch.int16)), (epi, od, b is None)
    y, y_ref, abs_sum, _ = _mx_case(mx, M, K, N, seed=M + 3 * K)
    assert_within(y.cpu().numpy(), y_ref, abs_sum, what="small linear")
