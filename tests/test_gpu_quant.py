"""GPU parity of the quantizers and the dequantizer against the CPU oracle (bit-exact)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O
from fp4_block_scaled_amd import synth
from _util import (activation_bits, dev_bits16, tile_mx, to_dev_bf16, unpack_fp4)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def mx():
    import fp4_block_scaled_amd as m
    assert torch.cuda.is_available()
    m.lib()
    return m


def _gpu_quant(mx, bits, fmt, sg=1.0):
    q = mx.quantize(to_dev_bf16(bits), fmt, sg)
    torch.cuda.synchronize()
    return q.codes.cpu().numpy(), q.scales.cpu().numpy()


ALL = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)


@pytest.mark.parametrize("fmt,elem", [("mxfp4", O.E2M1), ("mxfp8", O.E4M3)])
def test_mx_quantizer_exhaustive_bf16(mx, fmt, elem):
    """Every BF16 pattern (NaN and Inf included) under several block maxima."""
    anchors = [0x0000, 0x40C0, 0x3F80, 0x4040, 0x0180, 0x0080, 0x7F7F, 0x43E0, 0x0001]
    for a in anchors:
        block = np.zeros((len(ALL), 32), dtype=np.uint16)
        block[:, 0] = ALL
        block[:, 1] = a
        block[:, 5] = ALL[::-1]
        ref_c, ref_s = O.quantize_mx_bf16(block, elem)
        c, s = _gpu_quant(mx, block, fmt)
        np.testing.assert_array_equal(s, ref_s, err_msg=f"scales, anchor {a:#06x}")
        np.testing.assert_array_equal(c, ref_c, err_msg=f"codes, anchor {a:#06x}")


@pytest.mark.parametrize("fmt,elem", [("mxfp4", O.E2M1), ("mxfp8", O.E4M3)])
def test_mx_quantizer_exhaustive_over_scale_exponents(mx, fmt, elem):
    """Every BF16 pattern under block maxima 1.5 * 2^k swept across the exponent range: the
    element rounding runs on the hardware scaled conversion, so every scale exponent it can be
    given is checked against the oracle (q = |x| 2^-e covers [0, 8) / [0, 512) in each case)."""
    for E in range(1, 255, 6):
        block = np.zeros((len(ALL), 32), dtype=np.uint16)
        block[:, 0] = ALL
        block[:, 1] = (E << 7) | 0x40
        block[:, 9] = ALL[::-1] ^ 0x8000
        ref_c, ref_s = O.quantize_mx_bf16(block, elem)
        c, s = _gpu_quant(mx, block, fmt)
        np.testing.assert_array_equal(s, ref_s, err_msg=f"scales, anchor exponent {E}")
        np.testing.assert_array_equal(c, ref_c, err_msg=f"codes, anchor exponent {E}")


@pytest.mark.parametrize("name,fmt,elem", [("mxfp4_worked_blocks.json", "mxfp4", O.E2M1),
                                           ("mxfp8_worked_blocks.json", "mxfp8", O.E4M3)])
def test_mx_worked_blocks_on_gpu(mx, name, fmt, elem):
    blocks = json.load(open(os.path.join(GOLDEN, name)))["blocks"]
    for b in blocks:
        if "bits" in b:
            bits = np.asarray(b["bits"], dtype=np.uint16)
        else:
            bits = synth.bits16(torch.tensor(b["x"], dtype=torch.float64).to(torch.float32)
                                .to(torch.bfloat16))
        c, s = _gpu_quant(mx, bits[None, :], fmt)
        assert int(s[0, 0]) == b["scale"], b["name"]
        codes = unpack_fp4(c[0], 32) if elem == O.E2M1 else c[0]
        np.testing.assert_array_equal(codes, b["codes"], err_msg=b["name"])


def test_nv_worked_blocks_on_gpu(mx):
    g = json.load(open(os.path.join(GOLDEN, "nvfp4_worked_blocks.json")))
    for b in g["blocks"]:
        if "bits" in b:
            bits = np.asarray(b["bits"], dtype=np.uint16)
        else:
            bits = synth.bits16(torch.tensor(b["x"], dtype=torch.float64).to(torch.float32)
                                .to(torch.bfloat16))
        sg = b.get("global_scale", g["global_scale"])
        c, s = _gpu_quant(mx, bits[None, :], "nvfp4", sg)
        assert int(s[0, 0]) == b["scale"], b["name"]
        np.testing.assert_array_equal(unpack_fp4(c[0], 16), b["codes"], err_msg=b["name"])


# 1e-24: block scales whose D = sb * sg falls below the fused test's range (exact thresholds);
# 1e-30: a global scale outside the block-scale bracket's range (fp64 quotient); 1e20: large
@pytest.mark.parametrize("sg", [1.0, 40.0 / 2688.0, 0.5, 3.0 / 7.0, 1e-3, 0.0625 / 2688.0, 1e-24, 1e-30, 1e20])
def test_nv_quantizer_vs_oracle(mx, sg):
    sg = float(np.float32(sg))
    x = synth.activation_f32(4321, 512, 1024, 1.0, 0.01, 30.0)
    x[::5] *= 1e-3
    x[1::7] *= 40.0
    bits = synth.bits16(synth.to_bf16(x))
    ref_c, ref_s = O.quantize_nv_bf16(bits, sg)
    c, s = _gpu_quant(mx, bits, "nvfp4", sg)
    np.testing.assert_array_equal(s, ref_s)
    np.testing.assert_array_equal(c, ref_c)


def test_nv_quantizer_exhaustive_bf16(mx):
    sg = float(np.float32(40.0 / 2688.0))
    for a in (0x0000, 0x4220, 0x3F80, 0x4300):
        block = np.zeros((len(ALL), 16), dtype=np.uint16)
        block[:, 0] = ALL
        block[:, 1] = a
        block[:, 9] = ALL[::-1]
        ref_c, ref_s = O.quantize_nv_bf16(block, sg)
        c, s = _gpu_quant(mx, block, "nvfp4", sg)
        np.testing.assert_array_equal(s, ref_s, err_msg=f"anchor {a:#06x}")
        np.testing.assert_array_equal(c, ref_c, err_msg=f"anchor {a:#06x}")


@pytest.mark.parametrize("sg", [1.0, 0.75, 2.0 ** -10, 3.0 / 7.0, 40.0 / 2688.0])
def test_nv_quantizer_ties_and_near_ties(mx, sg):
    """Blocks built on the rounding midpoints: elements m * 2^k * sg with m an E2M1 midpoint or
    grid value, and a block maximum placed on or next to an E4M3 midpoint.  At a power-of-two or
    short global scale these are exact ties (the even code wins); at 3/7 and 40/2688 the BF16
    rounding leaves them within a few units in the last place of a midpoint on either side."""
    sg = float(np.float32(sg))
    rng = np.random.default_rng(4100)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.5, 1.0, 3.0, 4.0])
    n = 8192
    blk = rng.choice(mids, (n, 16)) * np.where(rng.integers(0, 2, (n, 16)) == 1, -1.0, 1.0)
    # block maximum 6 * s with s on an E4M3 value (exact block scale) or midpoint (a scale tie)
    e4m3_mid = np.array([1.0625, 1.1875, 1.3125, 1.4375, 1.5625, 1.6875, 1.8125, 1.9375])
    smax = np.where(rng.integers(0, 2, n) == 1, rng.choice(e4m3_mid, n), 1.0)
    blk[:, 0] = 6.0 * smax
    x = (blk * np.exp2(rng.integers(-8, 9, (n, 1))) * sg).astype(np.float32)
    bits = synth.bits16(synth.to_bf16(x)).reshape(-1, 256)
    ref_c, ref_s = O.quantize_nv_bf16(bits, sg)
    c, s = _gpu_quant(mx, bits, "nvfp4", sg)
    np.testing.assert_array_equal(s, ref_s)
    np.testing.assert_array_equal(c, ref_c)


@pytest.mark.parametrize("rows,cols,ld", [(1, 16, 16), (3, 96, 104), (257, 528, 536), (1000, 3072, 3072)])
def test_nv_quantizer_shapes_and_strides(mx, rows, cols, ld):
    sg = float(np.float32(40.0 / 2688.0))
    full = activation_bits(rows, ld, seed_base=7500 + cols, factor=30.0)
    x = to_dev_bf16(full)[:, :cols]
    q = mx.quantize(x, "nvfp4", sg)
    torch.cuda.synchronize()
    ref_c, ref_s = O.quantize_nv_bf16(np.ascontiguousarray(full[:, :cols]), sg)
    np.testing.assert_array_equal(q.scales.cpu().numpy(), ref_s)
    np.testing.assert_array_equal(q.codes.cpu().numpy(), ref_c)


@pytest.mark.parametrize("rows,cols,ld", [(1, 32, 32), (3, 96, 104), (257, 512, 512),
                                          (1000, 3072, 3072)])
@pytest.mark.parametrize("fmt,elem", [("mxfp4", O.E2M1), ("mxfp8", O.E4M3)])
def test_mx_quantizer_shapes_and_strides(mx, rows, cols, ld, fmt, elem):
    full = activation_bits(rows, ld, seed_base=7000 + cols)
    x = to_dev_bf16(full)[:, :cols]
    q = mx.quantize(x, fmt)
    torch.cuda.synchronize()
    ref_c, ref_s = O.quantize_mx_bf16(np.ascontiguousarray(full[:, :cols]), elem)
    np.testing.assert_array_equal(q.scales.cpu().numpy(), ref_s)
    np.testing.assert_array_equal(q.codes.cpu().numpy(), ref_c)


def test_quantizer_writes_nothing_past_its_outputs_and_is_deterministic(mx):
    rows, cols = 77, 640
    bits = activation_bits(rows, cols, seed_base=7100)
    x = to_dev_bf16(bits)
    codes = torch.full((rows * cols // 2 + 4096,), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((rows * cols // 32 + 4096,), 0xCD, dtype=torch.uint8, device="cuda")
    out = mx.QMatrix(codes[: rows * cols // 2].view(rows, cols // 2),
                     scales[: rows * cols // 32].view(rows, cols // 32), mx.MXFP4, rows, cols)
    mx.quantize(x, "mxfp4", out=out)
    first = (codes.clone(), scales.clone())
    mx.quantize(x, "mxfp4", out=out)
    torch.cuda.synchronize()
    assert torch.all(codes[rows * cols // 2:] == 0xAB)
    assert torch.all(scales[rows * cols // 32:] == 0xCD)
    assert torch.equal(first[0], codes) and torch.equal(first[1], scales)


def test_row_shards_quantize_identically(mx):
    bits = activation_bits(300, 1024, seed_base=7200)
    x = to_dev_bf16(bits)
    whole = mx.quantize(x, "mxfp4")
    for a, b in ((0, 1), (1, 129), (129, 300)):
        part = mx.quantize(x[a:b], "mxfp4")
        torch.cuda.synchronize()
        assert torch.equal(part.codes, whole.codes[a:b])
        assert torch.equal(part.scales, whole.scales[a:b])


@pytest.mark.parametrize("fmt,elem", [("mxfp4", O.E2M1), ("mxfp8", O.E4M3)])
def test_dequantize_mx_exact(mx, fmt, elem):
    bits = activation_bits(64, 1024, seed_base=7300)
    q = mx.quantize(to_dev_bf16(bits), fmt)
    y = mx.dequantize(q)
    torch.cuda.synchronize()
    ref = O.dequantize_mx(q.codes.cpu().numpy(), q.scales.cpu().numpy(), 1024, elem)
    np.testing.assert_array_equal(dev_bits16(y), O.bf16_rne_array(ref))
    # requantizing the dequantized tensor is the identity
    q2 = mx.quantize(y, fmt)
    torch.cuda.synchronize()
    assert torch.equal(q2.codes, q.codes) and torch.equal(q2.scales, q.scales)


def test_dequantize_nv(mx):
    sg = float(np.float32(40.0 / 2688.0))
    bits = activation_bits(64, 1024, seed_base=7400, factor=30.0)
    q = mx.quantize(to_dev_bf16(bits), "nvfp4", sg)
    y = mx.dequantize(q)
    torch.cuda.synchronize()
    ref = O.dequantize_nv(q.codes.cpu().numpy(), q.scales.cpu().numpy(), sg, 1024)
    np.testing.assert_array_equal(dev_bits16(y), O.bf16_rne_array(ref))


def test_absmax_and_global_scale(mx):
    bits = activation_bits(333, 640, seed_base=7500, factor=30.0)
    a = mx.absmax(to_dev_bf16(bits)).item()
    assert a == O.absmax_bf16(bits)
    assert mx.nvfp4_global_scale(a) == O.nv_global_scale(a)


@pytest.mark.parametrize("wl_name", ["wan_a14b_attn_75600x5120x5120",
                                     "wan_ti2v5b_w4a8_4290x3072x3072"])
def test_full_size_activation_quantizer(mx, wl_name):
    """The activation quantizer at the full workload size, every element against the oracle."""
    wl = synth.WORKLOADS[wl_name]
    bits = synth.bits16(synth.to_bf16(wl.activation()))
    fmt, elem = ("mxfp8", O.E4M3) if wl.fmt == "w4a8" else ("mxfp4", O.E2M1)
    c, s = _gpu_quant(mx, bits, fmt)
    ref_c, ref_s = O.quantize_mx_bf16(bits, elem)
    assert np.array_equal(s, ref_s)
    assert np.array_equal(c, ref_c)


def test_full_size_nvfp4_activation_quantizer(mx):
    wl = synth.WORKLOADS["wan_a14b_nvfp4_75600x5120x13824"]
    sg = O.nv_global_scale(wl.act_amax_static)
    bits = synth.bits16(synth.to_bf16(wl.activation()))
    c, s = _gpu_quant(mx, bits, "nvfp4", sg)
    ref_c, ref_s = O.quantize_nv_bf16(bits, sg)
    assert np.array_equal(s, ref_s)
    assert np.array_equal(c, ref_c)


# ---------------------------------------------------------------------------------------------
# tiled GEMM operand layout
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("rows,cols", [(300, 640), (1, 128), (256, 1024), (70, 384)])
@pytest.mark.parametrize("fmt,elem", [("mxfp4", O.E2M1), ("mxfp8", O.E4M3)])
def test_tiled_quantizer_is_the_tiled_oracle(mx, rows, cols, fmt, elem):
    bits = activation_bits(rows, cols, seed_base=15000 + rows + cols)
    ref_c, ref_s = O.quantize_mx_bf16(bits, elem)
    tc, ts = tile_mx(ref_c, ref_s, rows, cols, fp8=(fmt == "mxfp8"))
    x = to_dev_bf16(bits)
    q = mx.quantize(x, fmt, layout="tiled")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q.scales.cpu().numpy(), ts)
    np.testing.assert_array_equal(q.codes.cpu().numpy(), tc)
    # relayout both ways moves the same bytes
    back = mx.relayout(q)
    fwd = mx.relayout(mx.quantize(x, fmt))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(back.codes.cpu().numpy(), ref_c)
    np.testing.assert_array_equal(back.scales.cpu().numpy(), ref_s)
    np.testing.assert_array_equal(fwd.codes.cpu().numpy(), tc)
    np.testing.assert_array_equal(fwd.scales.cpu().numpy(), ts)


@pytest.mark.parametrize("fmt,elem", [("mxfp4", O.E2M1), ("mxfp8", O.E4M3)])
def test_tiled_quantizer_exhaustive_bf16(mx, fmt, elem):
    """Every BF16 pattern, four 32-element groups per row, through the tiled quantizer."""
    block = np.zeros((len(ALL), 32), dtype=np.uint16)
    block[:, 0] = ALL
    block[:, 1] = 0x40C0
    block[:, 7] = ALL[::-1]
    bits = block.reshape(len(ALL) // 4, 128)
    ref_c, ref_s = O.quantize_mx_bf16(bits, elem)
    tc, ts = tile_mx(ref_c, ref_s, bits.shape[0], 128, fp8=(fmt == "mxfp8"))
    q = mx.quantize(to_dev_bf16(bits), fmt, layout="tiled")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q.scales.cpu().numpy(), ts)
    np.testing.assert_array_equal(q.codes.cpu().numpy(), tc)


def test_tiled_outputs_write_nothing_past_their_buffers(mx):
    rows, cols = 37, 256
    x = to_dev_bf16(activation_bits(rows, cols, seed_base=15500))
    cb, sb = mx.tiled_bytes(rows, cols, "mxfp4")
    codes = torch.full((cb + 4096,), 0xA5, dtype=torch.uint8, device="cuda")
    scales = torch.full((sb + 4096,), 0x5A, dtype=torch.uint8, device="cuda")
    q = mx.QMatrix(codes[:cb], scales[:sb], mx.MXFP4, rows, cols, layout=mx.TILED)
    mx.quantize(x, out=q)
    torch.cuda.synchronize()
    assert torch.all(codes[cb:] == 0xA5) and torch.all(scales[sb:] == 0x5A)
