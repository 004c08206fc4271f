"""GPU parity of microscaled attention (MXFP4 Q/K, MXFP8 V and probabilities) and of the V^T
MXFP8 quantizer, against the oracle.

The V^T quantizer and the Q/K quantizer are compared bit for bit.  The attention output is
compared element by element with the oracle's fp64 result on the oracle's own quantized
operands, within

    bound + (2e-3 + nblk * 2^-23) * absacc + 1e-6

absacc = sum_j p^_j |v_jd| / l is the sum of |products| of the probabilities-times-V product,
a block-scaled GEMM, so the GEMM tolerance 2e-3 * sum |a w| applies to it; nblk * 2^-23
covers the fp32 rescale-and-add of o and l once per key block (nblk blocks) and the fp32
scores and exponentials (the FP4 score products are exact); 1e-6 absorbs results near zero
and probabilities below fp32's normal range.  bound is the oracle's worst case for
probabilities that quantize to a neighbouring E4M3 value (the GPU's p is the fp32 evaluation
of the same expression, so a p within rounding noise of an E4M3 rounding boundary, or of a
power of two that moves the group scale, may land on the other side).

Flips are rare (a relative noise of ~1e-7 against E4M3 steps of 2^-4..2^-3), so nearly every
element must also be within (2^-12 + nblk * 2^-23) * absacc + 1e-6 without the bound: 2^-12
is twice the accumulation error of the FP8 x FP8 scaled MFMA over one 64-key block as measured
through the W8A8 GEMM on a softmax block's probabilities (8.8e-5 of sum |p^ v^|; the matrix
core does not accumulate a block's products exactly in fp32).
"""
import numpy as np
import pytest
import torch

import oracle as O
from fp4_block_scaled_amd import synth
from _util import bf16_rne_of_f32, dev_bits16, sample_rows, split_exact, to_dev_bf16

pytestmark = pytest.mark.gpu

D = 128
KVB = 64


@pytest.fixture(scope="module")
def mx():
    import fp4_block_scaled_amd as m
    assert torch.cuda.is_available()
    m.lib()
    return m


def _bits(seed, shape, sigma):
    return synth.bits16(synth.to_bf16(synth.normal_f32(seed, shape, sigma)))


def _tol(bnd, ab, S, with_bound=True):
    nblk = (S + KVB - 1) // KVB
    if with_bound:
        return bnd + (2e-3 + nblk * 2.0 ** -23) * ab + 1e-6
    return (2.0 ** -12 + nblk * 2.0 ** -23) * ab + 1e-6


def _compare(o_gpu, ref, bnd, ab, S, what, extra=0.0, flip_frac=0.02):
    err = np.abs(o_gpu.astype(np.float64) - ref)
    tol = _tol(bnd, ab, S) + extra
    bad = err > tol
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance, first "
                           f"{np.argwhere(bad)[:4].tolist()}, max err/tol {np.max(err / tol):.3g}")
    tight = err > _tol(bnd, ab, S, with_bound=False) + extra
    frac = float(np.mean(tight))
    print(f"{what}: max err/tol {np.max(err / tol):.3g}, beyond the no-flip tolerance: {frac:.2e}")
    assert frac <= flip_frac


def _blocked(vtc, vts):
    """The oracle's V^T MXFP8 ([BH, D, Sp] codes, [BH, D, Sp/32] scales) in the library's
    key-block-major layout ([BH, Sp/64, D, 64], [BH, Sp/64, D, 2])."""
    BH, D_, Sp = vtc.shape
    nb = Sp // KVB
    return (np.ascontiguousarray(vtc.reshape(BH, D_, nb, KVB).transpose(0, 2, 1, 3)),
            np.ascontiguousarray(vts.reshape(BH, D_, nb, 2).transpose(0, 2, 1, 3)))


def _oracle_operands(q_bits, k_bits, v_bits, BH, S):
    qc, qs = O.quantize_mx_bf16(q_bits)
    kc, ks = O.quantize_mx_bf16(k_bits)
    vtc, vts = O.quantize_vt_mx8(v_bits, BH, S, D, KVB)
    return qc, qs, kc, ks, vtc, vts


@pytest.mark.parametrize("BH,S,D_", [(2, 100, 128), (3, 64, 64), (1, 1, 32), (2, 257, 256), (1, 1000, 96)])
def test_quantize_vt_bit_exact(mx, BH, S, D_):
    v_bits = _bits(31000 + S, (BH, S, D_), 1.0)
    v_bits[0, 0, :4] = 0  # a zero run inside a group
    codes, scales = mx.quantize_vt(to_dev_bf16(v_bits))
    torch.cuda.synchronize()
    rc, rs = _blocked(*O.quantize_vt_mx8(v_bits, BH, S, D_, KVB))
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)


def test_quantize_vt_strided_view_and_extremes(mx):
    """A transposed view of an [S, H, D] projection (head stride D, row stride H * D), with
    large, tiny and zero values in it."""
    S, H = 150, 3
    x = synth.normal_f32(31500, (S, H * D), 1.0)
    x[:7, :40] *= 3000.0
    x[20:60, 128:200] *= 1e-30
    x[100:140, 256:300] = 0.0
    v_bits = synth.bits16(synth.to_bf16(x))
    v = to_dev_bf16(v_bits).view(S, H, D).transpose(0, 1)
    codes, scales = mx.quantize_vt(v)
    torch.cuda.synchronize()
    ref_in = np.ascontiguousarray(v_bits.reshape(S, H, D).transpose(1, 0, 2))
    rc, rs = _blocked(*O.quantize_vt_mx8(ref_in, H, S, D, KVB))
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("BH,S,sigma,scale", [
    (2, 200, 1.0, D ** -0.5),   # ragged key block and query block
    (1, 64, 1.0, D ** -0.5),    # one whole key block
    (3, 1, 1.0, D ** -0.5),     # a single key: out = v^ exactly
    (1, 129, 3.0, D ** -0.5),   # sharp softmax (scores spread over ~100 in log2 units)
    (2, 384, 1.5, 0.2),
    (1, 1000, 1.0, D ** -0.5),  # 16 key blocks
    (1, 63, 1.0, D ** -0.5),    # one key short of a block
    (1, 65, 1.0, D ** -0.5),    # one key past a block
    (2, 128, 2.0, D ** -0.5),   # exactly one query block per head
])
def test_attention_vs_oracle(mx, BH, S, sigma, scale):
    q_bits = _bits(32000 + S, (BH * S, D), sigma)
    k_bits = _bits(32100 + S, (BH * S, D), sigma)
    v_bits = _bits(32200 + S, (BH * S, D), 1.0)
    qc, qs, kc, ks, vtc, vts = _oracle_operands(q_bits, k_bits, v_bits, BH, S)
    qg = mx.quantize(to_dev_bf16(q_bits), "mxfp4")
    kg = mx.quantize(to_dev_bf16(k_bits), "mxfp4")
    vt = mx.quantize_vt(to_dev_bf16(v_bits).view(BH, S, D))
    o = mx.attention(qg, kg, vt, heads=BH, softmax_scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(qg.codes.cpu().numpy(), qc) and np.array_equal(kg.scales.cpu().numpy(), ks)
    ref, bnd, ab = O.attention_mx(qc, qs, kc, ks, vtc, vts, BH, S, D, KVB, scale)
    _compare(o.cpu().numpy().reshape(BH * S, D), ref, bnd, ab, S, f"attention BH={BH} S={S}")


# Scores of 128 key slots (two blocks of 64): groups 1 and 3 sit 2^24 and more below their
# block's maximum, and their V values are 2^24 larger than those of groups 0 and 2, so their
# products carry most of the output.  Keys 120..127 are past S_kv (masked).
_GS = np.full(128, -6.0)
_GS[:16] = [0, -0.5, -1, -1.5, -2, -3, -4, -6, -8, -0.25, -0.75, -2.5, -3.5, -5, -7, -10]
_GS[32:48] = [-24, -24.5, -25, -26, -27, -28, -30, -32, -36, -24.25, -25.5, -29, -33, -40, -26.5, -27.5]
_GS[48:64] = -31.0
_GS[64:80] = [-0.5, -1, -1.5, -2, -3, -0.25, -0.75, -4, -5, -6, -2.5, -3.5, -7, -9, -12, -16]
_GS[96:120] = -27.0
_GS[96:104] = [-26, -25, -30, -24.5, -33, -28, -24.75, -36]


def test_probability_groups_of_32_keys(mx):
    """The probabilities are quantized to MXFP8 in groups of 32 keys, each group with its own
    scale.  Scores are exact (Q and K hold +-2^a or +-1.5 * 2^a alone in their 32-element blocks,
    softmax_scale = ln 2 so that c = 1), groups 1 and 3 lie 2^24 and more below their 64-key
    block's maximum with V 2^24 larger and of one sign: a scale per 64 keys (or one shared by the
    wrong groups) would zero those probabilities and remove most of the output.  F32 out against
    the oracle; and the oracle without groups 1 and 3 lies outside the tolerance everywhere, so
    the test can fail."""
    BH, Sq, Skv = 1, 40, 120
    q = np.zeros((Sq, D), dtype=np.float32)
    q[:, [0, 32, 64]] = 1.0
    k = np.zeros((Skv, D), dtype=np.float32)
    for j in range(Skv):
        k[j, [0, 32, 64]] = split_exact(float(_GS[j]))
    v = synth.normal_f32(37000, (Skv, D), 1.0)
    far = np.zeros(Skv, dtype=bool)
    far[32:64] = far[96:] = True
    v[far] = np.abs(v[far]) * 2.0 ** 24  # one sign: the far products add up
    q_bits, k_bits, v_bits = (synth.bits16(synth.to_bf16(x)) for x in (q, k, v))
    # c = softmax_scale * log2(e) is exactly 1 on both sides: the oracle divides ln 2 by ln 2
    # in fp64, the kernel rounds fp32(ln 2) * log2(e) to binary32, which is 1.0
    scale = float(np.log(2.0))
    qc, qs = O.quantize_mx_bf16(q_bits)
    kc, ks = O.quantize_mx_bf16(k_bits)
    # the scores are exact: the quantized Q and K hold the values given above
    assert np.array_equal(O.dequantize_mx(kc, ks, D)[:, [0, 32, 64]].sum(axis=1), _GS[:Skv])
    vtc, vts = O.quantize_vt_mx8(v_bits, BH, Skv, D, KVB)
    o = mx.attention(mx.quantize(to_dev_bf16(q_bits), "mxfp4"), mx.quantize(to_dev_bf16(k_bits), "mxfp4"),
                     mx.quantize_vt(to_dev_bf16(v_bits).view(BH, Skv, D)), BH, softmax_scale=scale,
                     out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref, bnd, ab = O.attention_mx(qc, qs, kc, ks, vtc, vts, BH, Sq, D, KVB, scale, S_kv=Skv)
    _compare(o.cpu().numpy().reshape(Sq, D), ref, bnd, ab, Skv, "32-key probability groups", flip_frac=0.05)
    vtc_near = vtc.copy()
    vtc_near[:, :, far.nonzero()[0]] = 0  # the far groups' products removed
    ablated, _, _ = O.attention_mx(qc, qs, kc, ks, vtc_near, vts, BH, Sq, D, KVB, scale, S_kv=Skv)
    assert np.all(np.abs(ablated - ref) > _tol(bnd, ab, Skv))


# Scores of one 64-key block for the exact probability test: group 0 holds the row maximum
# (p = 1, scale 2^-8, so nothing there can pass 448 * 2^-8); group 1's largest p is 2^-1/16
# = 0.9576, scale 2^-9, so p / 2^-9 = 490.3 and 469.5 (keys 32, 33) lie past the largest E4M3
# value and must saturate to 448, 449.6 (key 34) rounds to 448, and 430.5, 394.8, 362.0 round to
# 416, 384, 352; none lies near a rounding boundary.
_SAT = np.full(64, -8.0)
_SAT[:12] = [0, -0.0625, -0.125, -0.1875, -0.25, -0.375, -0.5, -1, -1.5, -2, -3, -6]
_SAT[32:44] = [-0.0625, -0.125, -0.1875, -0.25, -0.375, -0.5, -1, -1.5, -2, -3, -6, -12]


def test_probability_codes_exact_with_saturation(mx):
    """The GPU's quantized probabilities read off exactly: exact scores (Q and K hold +-2^a or
    +-1.5 * 2^a alone in their blocks, softmax_scale = ln 2 so that c = 1) and V one-hot (key j
    carries 1 in head-dim column j, exact in MXFP8), so out[d] = p^_d / l, and key 0 (p = 1,
    code 256 * 2^-8, exact) gives p^_d = out[d] / out[0].  Expected codes: p = 2^s in fp64, the
    group scale floor(log2 max p) - 8, p / 2^scale saturated at 448 and rounded by torch's E4M3
    cast.  Two keys of group 1 pass the largest E4M3 value, so a conversion without saturation
    (E4M3 has no infinity: it gives NaN there) fails."""
    BH, Sq, Skv = 1, 32, 64
    q = np.zeros((Sq, D), dtype=np.float32)
    q[:, [0, 32, 64]] = 1.0
    k = np.zeros((Skv, D), dtype=np.float32)
    for j in range(Skv):
        k[j, [0, 32, 64]] = split_exact(float(_SAT[j]))
    v = np.zeros((Skv, D), dtype=np.float32)
    v[np.arange(Skv), np.arange(Skv)] = 1.0
    q_bits, k_bits, v_bits = (synth.bits16(synth.to_bf16(x)) for x in (q, k, v))
    o = mx.attention(mx.quantize(to_dev_bf16(q_bits), "mxfp4"), mx.quantize(to_dev_bf16(k_bits), "mxfp4"),
                     mx.quantize_vt(to_dev_bf16(v_bits).view(BH, Skv, D)), BH,
                     softmax_scale=float(np.log(2.0)), out_dtype=torch.float32)
    torch.cuda.synchronize()
    o = o.cpu().numpy().reshape(Sq, D).astype(np.float64)
    assert np.all(o[:, Skv:] == 0.0)
    got = o[:, :Skv] / o[:, :1]
    p = 2.0 ** _SAT
    want = np.empty(Skv)
    for g in range(2):
        grp = p[32 * g:32 * g + 32]
        e = np.floor(np.log2(grp.max())) - 8
        qv = np.minimum(grp / 2.0 ** e, 448.0)
        want[32 * g:32 * g + 32] = torch.from_numpy(qv).float().to(torch.float8_e4m3fn).double().numpy() * 2.0 ** e
    assert (p[32:34] / 2.0 ** -9 > 464).all()  # the saturating keys are there
    np.testing.assert_allclose(got, np.broadcast_to(want, got.shape), rtol=2.0 ** -20, atol=0)


def test_single_key_is_v_exactly(mx):
    """With one key every probability is 1 (quantized exactly), so out = v^ for every query."""
    BH, S = 2, 1
    q_bits = _bits(33000, (BH * S, D), 2.0)
    k_bits = _bits(33001, (BH * S, D), 2.0)
    v_bits = _bits(33002, (BH * S, D), 1.0)
    vt = mx.quantize_vt(to_dev_bf16(v_bits).view(BH, S, D))
    o = mx.attention(mx.quantize(to_dev_bf16(q_bits), "mxfp4"), mx.quantize(to_dev_bf16(k_bits), "mxfp4"),
                     vt, heads=BH, out_dtype=torch.float32)
    torch.cuda.synchronize()
    vtc, vts = O.quantize_vt_mx8(v_bits, BH, S, D, KVB)
    vhat = np.vectorize(O.e4m3_value)(vtc[:, :, 0]) * np.vectorize(O.e8m0_value)(vts[:, :, 0])
    np.testing.assert_array_equal(o.cpu().numpy().reshape(BH, D).astype(np.float64), vhat)


def test_attention_bf16_out_and_shd_layout(mx):
    """Heads interleaved in the row ([S, H * 128], one batch of the projections) and BF16 out:
    the BF16 result is the RNE of a value within the F32 tolerance."""
    S, H, scale = 150, 3, D ** -0.5
    q_bits = _bits(34000, (S, H * D), 1.2)
    k_bits = _bits(34001, (S, H * D), 1.2)
    v_bits = _bits(34002, (S, H * D), 1.0)
    heads = lambda b: np.ascontiguousarray(b.reshape(S, H, D).transpose(1, 0, 2)).reshape(H * S, D)
    qc, qs, kc, ks, vtc, vts = _oracle_operands(heads(q_bits), heads(k_bits), heads(v_bits), H, S)
    vt = mx.quantize_vt(to_dev_bf16(v_bits).view(S, H, D).transpose(0, 1))
    o = mx.attention(mx.quantize(to_dev_bf16(q_bits), "mxfp4"), mx.quantize(to_dev_bf16(k_bits), "mxfp4"),
                     vt, heads=H, layout="shd")
    torch.cuda.synchronize()
    assert np.array_equal(vt[0].cpu().numpy(), _blocked(vtc, vts)[0])
    ref, bnd, ab = O.attention_mx(qc, qs, kc, ks, vtc, vts, H, S, D, KVB, scale)
    got = O.bf16_values(dev_bits16(o)).reshape(S, H, D).transpose(1, 0, 2).reshape(H * S, D)
    _compare(got, ref, bnd, ab, S, "attention shd bf16", extra=2.0 ** -8 * np.abs(ref))


@pytest.mark.parametrize("name", ["wan_a14b_attn_mx_75600x40x128", "wan_ti2v5b_attn_mx_4290x24x128"])
def test_full_size_wan_attention(mx, name):
    """Full Wan2.2 self-attention shapes (A14B at 720p: 75600 tokens x 40 heads, as the benchmark
    runs it; TI2V-5B: 4290 tokens x 24 heads), in the projections' layout: sampled queries of
    three heads (including the last, partial query block; the last key block holds 16 / 2 keys)
    in F32 against the oracle, the BF16 output as the RNE of the F32 one, and the V^T codes of
    those heads bit for bit."""
    wl = synth.WORKLOADS[name]
    S, H = wl.M, wl.extra["heads"]
    q, k, v = wl.qkv()
    bits = [synth.bits16(synth.to_bf16(x)) for x in (q, k, v)]
    del q, k, v
    qd, kd, vd = (to_dev_bf16(b) for b in bits)
    qg, kg = mx.quantize(qd, "mxfp4"), mx.quantize(kd, "mxfp4")
    vt = mx.quantize_vt(vd.view(S, H, D).transpose(0, 1))
    o = mx.attention(qg, kg, vt, heads=H, layout="shd", out_dtype=torch.float32)
    o16 = mx.attention(qg, kg, vt, heads=H, layout="shd")
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([sample_rows(S, 24), [0, S - 80, S - 1]]))
    for h in (0, H // 2 - 3, H - 1):
        hb = [np.ascontiguousarray(b[:, h * D:(h + 1) * D]) for b in bits]
        qc, qs, kc, ks, vtc, vts = _oracle_operands(hb[0], hb[1], hb[2], 1, S)
        bc, bs = _blocked(vtc, vts)
        assert np.array_equal(vt[0][h].cpu().numpy(), bc[0]) and np.array_equal(vt[1][h].cpu().numpy(), bs[0])
        ref, bnd, ab = O.attention_mx(qc, qs, kc, ks, vtc, vts, 1, S, D, KVB, D ** -0.5, qrows=rows)
        idx = torch.from_numpy(rows).cuda()
        got = o[idx, h * D:(h + 1) * D].cpu().numpy()
        _compare(got, ref, bnd, ab, S, f"full-size head {h}", flip_frac=0.05)
        # the BF16 output is the RNE of the F32 one
        np.testing.assert_array_equal(dev_bits16(o16[idx, h * D:(h + 1) * D]), bf16_rne_of_f32(got))


def test_head_and_row_strides_through_the_c_abi(mx):
    """Heads spaced apart in memory (a head stride beyond S rows) for Q/K and the output, called
    through the C ABI directly: bit-identical to the dense call."""
    import ctypes
    BH, S, pad = 3, 150, 26
    q_bits = _bits(35000, (BH, S, D), 1.0)
    k_bits = _bits(35001, (BH, S, D), 1.0)
    v_bits = _bits(35002, (BH, S, D), 1.0)
    dense = mx.attention(mx.quantize(to_dev_bf16(q_bits.reshape(BH * S, D)), "mxfp4"),
                         mx.quantize(to_dev_bf16(k_bits.reshape(BH * S, D)), "mxfp4"),
                         mx.quantize_vt(to_dev_bf16(v_bits)), BH, out_dtype=torch.float32)
    padded = lambda b: np.concatenate([b, np.zeros((BH, pad, D), np.uint16)], axis=1).reshape(BH * (S + pad), D)
    qp = mx.quantize(to_dev_bf16(padded(q_bits)), "mxfp4")
    kp = mx.quantize(to_dev_bf16(padded(k_bits)), "mxfp4")
    vt = mx.quantize_vt(to_dev_bf16(v_bits))
    out = torch.full((BH, S + pad, D), float("nan"), dtype=torch.float32, device="cuda")
    hs = (S + pad) * D
    st = mx.lib().mx_attention(qp.codes.data_ptr(), qp.scales.data_ptr(), D, hs, kp.codes.data_ptr(),
                               kp.scales.data_ptr(), D, hs, vt[0].data_ptr(), vt[1].data_ptr(), BH, S, S,
                               D, ctypes.c_float(D ** -0.5), 1, out.data_ptr(), D, hs,
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0
    assert torch.equal(out[:, :S], dense)
    assert torch.isnan(out[:, S:]).all()  # rows past S untouched


@pytest.mark.parametrize("BH,Sq,Skv,sigma", [
    (2, 300, 77, 1.0),    # more queries than keys, ragged key block
    (1, 64, 512, 1.0),    # eight key blocks for one query block
    (3, 10, 1, 1.0),      # a single key: out = v^
    (2, 129, 200, 2.0),   # sharper softmax
])
def test_cross_attention_vs_oracle(mx, BH, Sq, Skv, sigma):
    """Queries and keys / values of different lengths (the second attention layer of the DiT
    attends to the conditioning context)."""
    q_bits = _bits(36000 + Sq, (BH * Sq, D), sigma)
    k_bits = _bits(36100 + Skv, (BH * Skv, D), sigma)
    v_bits = _bits(36200 + Skv, (BH * Skv, D), 1.0)
    qc, qs = O.quantize_mx_bf16(q_bits)
    kc, ks = O.quantize_mx_bf16(k_bits)
    vtc, vts = O.quantize_vt_mx8(v_bits, BH, Skv, D, KVB)
    o = mx.attention(mx.quantize(to_dev_bf16(q_bits), "mxfp4"), mx.quantize(to_dev_bf16(k_bits), "mxfp4"),
                     mx.quantize_vt(to_dev_bf16(v_bits).view(BH, Skv, D)), BH, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref, bnd, ab = O.attention_mx(qc, qs, kc, ks, vtc, vts, BH, Sq, D, KVB, D ** -0.5, S_kv=Skv)
    _compare(o.cpu().numpy().reshape(BH * Sq, D), ref, bnd, ab, Skv, f"cross-attention {Sq}x{Skv}")


@pytest.mark.parametrize("name", ["wan_a14b_attn_mx_75600x40x128", "wan_ti2v5b_attn_mx_4290x24x128"])
def test_full_size_wan_cross_attention(mx, name):
    """The workload's queries against 512 context tokens (keys and values N(0,1), seeded), in the
    projections' layout with F32 out: sampled queries of three heads against the oracle."""
    wl = synth.WORKLOADS[name]
    Sq, H, Skv = wl.M, wl.extra["heads"], 512
    q_bits = synth.bits16(synth.to_bf16(wl.qkv(Sq)[0]))
    k_bits = _bits(wl.seed_base + 21, (Skv, H * D), 1.0)
    v_bits = _bits(wl.seed_base + 22, (Skv, H * D), 1.0)
    vt = mx.quantize_vt(to_dev_bf16(v_bits).view(Skv, H, D).transpose(0, 1))
    o = mx.attention(mx.quantize(to_dev_bf16(q_bits), "mxfp4"), mx.quantize(to_dev_bf16(k_bits), "mxfp4"),
                     vt, heads=H, layout="shd", out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([sample_rows(Sq, 24), [0, Sq - 1]]))
    for h in (0, H // 2 - 3, H - 1):
        hq = np.ascontiguousarray(q_bits[:, h * D:(h + 1) * D])
        hk = np.ascontiguousarray(k_bits[:, h * D:(h + 1) * D])
        hv = np.ascontiguousarray(v_bits[:, h * D:(h + 1) * D])
        qc, qs = O.quantize_mx_bf16(hq)
        kc, ks = O.quantize_mx_bf16(hk)
        vtc, vts = O.quantize_vt_mx8(hv, 1, Skv, D, KVB)
        ref, bnd, ab = O.attention_mx(qc, qs, kc, ks, vtc, vts, 1, Sq, D, KVB, D ** -0.5, qrows=rows, S_kv=Skv)
        got = o[torch.from_numpy(rows).cuda(), h * D:(h + 1) * D].cpu().numpy()
        _compare(got, ref, bnd, ab, Skv, f"full-size cross head {h}", flip_frac=0.05)
