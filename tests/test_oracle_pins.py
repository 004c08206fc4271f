"""Pins of the CPU oracle against what the pages and the mathematics fix (CPU only).

Each test checks the oracle against something other than itself: values stated on the pages
(golden fixtures), hand-derived worked examples, exhaustive brute-force searches written
independently here (argmin over the value grid, exact rational arithmetic), and library routines
(torch's float8/bfloat16 conversions, torch's tanh-GELU, numpy matmul).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from fp4_block_scaled_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bf16_bits_exact(values):
    """float values -> BF16 bit patterns, asserting each value is exactly representable."""
    t = torch.tensor(values, dtype=torch.float64)
    b = t.to(torch.float32).to(torch.bfloat16)
    assert torch.equal(b.to(torch.float64), t) and torch.equal(torch.signbit(b), torch.signbit(t))
    return b.view(torch.int16).numpy().view(np.uint16)


def _unpack(packed, n):
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (n,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


E2M1_GRID = np.array(_golden("e2m1_grid.json")["magnitudes"], dtype=np.float64)
# E4M3 magnitudes 0..126 from torch's float8_e4m3fn decoding (library, independent of the oracle)
E4M3_GRID = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(
    torch.float64).numpy()


# ---------------------------------------------------------------------------------------------
# element formats
# ---------------------------------------------------------------------------------------------
def test_e2m1_decode_is_the_stated_grid():
    g = _golden("e2m1_grid.json")
    for c in range(8):
        assert O.e2m1_value(c) == g["magnitudes"][c]
        neg = O.e2m1_value(c | g["sign_bit"])
        assert neg == -g["magnitudes"][c] and math.copysign(1.0, neg) == -1.0
    vals = sorted({O.e2m1_value(c) for c in range(16)})
    assert len(vals) == 15  # +0 and -0 compare equal: 16 codes, 15 distinct reals


def test_e4m3_decode_matches_torch():
    ref = torch.arange(0, 256, dtype=torch.int32).to(torch.uint8).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        v = O.e4m3_value(b)
        if b in (0x7F, 0xFF):
            assert math.isnan(v)
        else:
            assert v == ref[b], b
    assert O.e4m3_value(0x7E) == 448.0 and O.e4m3_value(0x01) == 2.0 ** -9


def test_e8m0_decode_is_power_of_two():
    for b in range(255):
        assert O.e8m0_value(b) == 2.0 ** (b - 127)
    assert math.isnan(O.e8m0_value(255))


def _nearest_even(q, grid):
    """Independent RNE: argmin distance over the grid, ties to the even index; saturates."""
    d = np.abs(q[:, None] - grid[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    first = cand.argmax(axis=1)
    two = cand.sum(axis=1) == 2
    return np.where(two & (first % 2 == 1), first + 1, first)


def test_e2m1_rne_bruteforce_dense():
    q = np.concatenate([np.arange(0, 8 * 256 + 1) / 256.0,
                        np.random.default_rng(0).uniform(0, 9, 20000)])
    ref = _nearest_even(q, E2M1_GRID)
    got = np.array([O.e2m1_rne_mag(float(v)) for v in q])
    np.testing.assert_array_equal(got, ref)


def test_e4m3_rne_matches_torch_conversion():
    # all midpoints and representable points below saturation, plus random fp32 values
    mags = E4M3_GRID
    mids = (mags[:-1] + mags[1:]) / 2
    rng = np.random.default_rng(1)
    rand = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(460.0), 20000)).astype(np.float32)
    q = np.concatenate([mags, mids, rand.astype(np.float64)])
    q = q[q < 448.0 + 8.0]          # torch turns >= 464 into NaN; saturation tested below
    tq = torch.tensor(q, dtype=torch.float32)
    assert torch.equal(tq.to(torch.float64), torch.tensor(q))  # fp32-exact inputs
    ref = tq.to(torch.float8_e4m3fn).view(torch.uint8).numpy() & 0x7F
    got = np.array([O.e4m3_rne_mag(float(v)) for v in q])
    np.testing.assert_array_equal(got, ref)
    for v in (464.0, 480.0, 1e6):
        assert O.e4m3_rne_mag(v) == 0x7E  # saturate, never the NaN code


def test_bf16_rne_matches_torch_and_ties():
    rng = np.random.default_rng(2)
    f = np.concatenate([rng.standard_normal(5000), rng.standard_normal(500) * 1e-39,
                        rng.standard_normal(500) * 1e37]).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([O.bf16_rne(float(v)) for v in f], dtype=np.uint16)
    np.testing.assert_array_equal(got, ref)
    # exact ties in fp64 beyond fp32 precision: 1 + 2^-8 -> 1 (even), 1 + 3*2^-8 -> 1 + 2^-6
    assert O.bf16_rne(1.0 + 2.0 ** -8) == 0x3F80
    assert O.bf16_rne(1.0 + 3 * 2.0 ** -8) == 0x3F82
    assert O.bf16_rne(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81  # just above the tie
    assert O.bf16_rne(-0.0) == 0x8000
    assert O.bf16_rne(3.5e38) == 0x7F80


# ---------------------------------------------------------------------------------------------
# worked examples
# ---------------------------------------------------------------------------------------------
def _block_bits(b):
    return np.asarray(b["bits"], dtype=np.uint16) if "bits" in b else _bf16_bits_exact(b["x"])


@pytest.mark.parametrize("b", _golden("mxfp4_worked_blocks.json")["blocks"], ids=lambda b: b["name"])
def test_mxfp4_worked_blocks(b):
    bits = _block_bits(b)[None, :]
    codes, scales = O.quantize_mx_bf16(bits, O.E2M1)
    assert int(scales[0, 0]) == b["scale"]
    np.testing.assert_array_equal(_unpack(codes[0], 32), b["codes"])
    if "packed" in b:
        np.testing.assert_array_equal(codes[0], b["packed"])
    assert codes.shape == (1, 16)  # two codes per byte


@pytest.mark.parametrize("b", _golden("mxfp8_worked_blocks.json")["blocks"], ids=lambda b: b["name"])
def test_mxfp8_worked_blocks(b):
    bits = _block_bits(b)[None, :]
    codes, scales = O.quantize_mx_bf16(bits, O.E4M3)
    assert int(scales[0, 0]) == b["scale"]
    np.testing.assert_array_equal(codes[0], b["codes"])


@pytest.mark.parametrize("b", _golden("nvfp4_worked_blocks.json")["blocks"], ids=lambda b: b["name"])
def test_nvfp4_worked_blocks(b):
    bits = _block_bits(b)[None, :]
    sg = b.get("global_scale", _golden("nvfp4_worked_blocks.json")["global_scale"])
    codes, scales = O.quantize_nv_bf16(bits, sg)
    assert int(scales[0, 0]) == b["scale"]
    np.testing.assert_array_equal(_unpack(codes[0], 16), b["codes"])
    if "packed" in b:
        np.testing.assert_array_equal(codes[0], b["packed"])


# ---------------------------------------------------------------------------------------------
# exhaustive brute force over every finite BF16 value
# ---------------------------------------------------------------------------------------------
_ALL_BF16 = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
_FINITE_BF16 = _ALL_BF16[(_ALL_BF16 & 0x7F80) != 0x7F80]


def _mx_brute(x_f64, anchor, emax, grid, sign_shift):
    amax = np.maximum(np.abs(x_f64), abs(anchor))
    _, ex = np.frexp(amax)
    e = np.where(amax == 0, -127, ex - 1 - emax)
    e = np.clip(e, -127, 127)
    q = np.ldexp(np.abs(x_f64), -e)
    idx = _nearest_even(q, grid)
    return (idx | (np.signbit(x_f64).astype(np.int64) << sign_shift)).astype(np.uint8), e + 127


@pytest.mark.parametrize("anchor", [0.0, 6.0, 1.0, 3.0, 2.0 ** -124, 2.0 ** -126, 1.5 * 2.0 ** 100,
                                    2.0 ** 127])
@pytest.mark.parametrize("elem", [O.E2M1, O.E4M3])
def test_mx_quantize_exhaustive_bf16(anchor, elem):
    x = O.bf16_values(_FINITE_BF16)
    n = len(x)
    abits = _bf16_bits_exact([anchor])[0]
    block = np.zeros((n, 32), dtype=np.uint16)
    block[:, 0] = _FINITE_BF16
    block[:, 1] = abits
    codes, scales = O.quantize_mx_bf16(block, elem)
    if elem == O.E2M1:
        got = _unpack(codes, 32)
        ref, sref = _mx_brute(x, anchor, 2, E2M1_GRID, 3)
        ref_a, _ = _mx_brute(np.full(n, anchor), np.abs(x), 2, E2M1_GRID, 3)
    else:
        got = codes
        ref, sref = _mx_brute(x, anchor, 8, E4M3_GRID, 7)
        ref_a, _ = _mx_brute(np.full(n, anchor), np.abs(x), 8, E4M3_GRID, 7)
    np.testing.assert_array_equal(scales[:, 0], sref)
    np.testing.assert_array_equal(got[:, 0], ref)
    np.testing.assert_array_equal(got[:, 1], ref_a)
    assert np.all(got[:, 2:] == 0)


# ---------------------------------------------------------------------------------------------
# exact rational brute force for NVFP4 (any global scale) and MX
# ---------------------------------------------------------------------------------------------
_E2M1_F = [Fraction(v) for v in E2M1_GRID]
_E4M3_F = [Fraction(float(v)) for v in E4M3_GRID]


def _rne_pick(q, mags):
    if q >= mags[-1]:
        return len(mags) - 1
    for i in range(len(mags) - 1):
        lo, hi = mags[i], mags[i + 1]
        if q <= hi:
            if q - lo < hi - q:
                return i
            if q - lo > hi - q:
                return i + 1
            return i if i % 2 == 0 else i + 1
    raise AssertionError


def _nv_ref(xs, sg):
    sgf = Fraction(float(np.float32(sg)))
    fx = [Fraction(float(v)) for v in xs]
    amax = max(abs(v) for v in fx)
    si = _rne_pick(amax / (6 * sgf), _E4M3_F)
    sb = _E4M3_F[si]
    codes = []
    for v, raw in zip(fx, xs):
        s = 8 if math.copysign(1.0, raw) < 0 else 0
        codes.append(s | (0 if sb == 0 else _rne_pick(abs(v) / (sb * sgf), _E2M1_F)))
    return codes, si


def _blocks_for_nv(nblk, seed):
    x = synth.activation_f32(seed, nblk, 16, 1.0, 0.1, 30.0)
    x[::7] *= 1e-3
    x[::11] *= 50.0
    return synth.bits16(synth.to_bf16(x))


@pytest.mark.parametrize("sg", [1.0, 40.0 / 2688.0, 0.5, 3.0 / 7.0, 1e-3])
def test_nvfp4_exact_rational_bruteforce(sg):
    sg32 = float(np.float32(sg))
    bits = _blocks_for_nv(64, 77)
    codes, scales = O.quantize_nv_bf16(bits, sg32)
    got = _unpack(codes, 16)
    xs = O.bf16_values(bits)
    for r in range(bits.shape[0]):
        ref_codes, ref_s = _nv_ref(xs[r], sg32)
        assert int(scales[r, 0]) == ref_s, r
        np.testing.assert_array_equal(got[r], ref_codes)


def test_nv_global_scale_is_rounded_quotient():
    for amax in (40.0, 1.0, 0.046875, 123.5, 2.0 ** -100):
        exp = Fraction(amax) / 2688
        got = Fraction(O.nv_global_scale(amax))
        # binary32 rounding of the exact quotient: nearest among neighbours
        f = np.float32(float(exp))
        cands = [np.nextafter(f, np.float32(0)), f, np.nextafter(f, np.float32(np.inf))]
        best = min(cands, key=lambda c: abs(Fraction(float(c)) - exp))
        assert got == Fraction(float(best))
    assert O.nv_global_scale(0.0) == 1.0


# ---------------------------------------------------------------------------------------------
# invariants of the scale rule
# ---------------------------------------------------------------------------------------------
def _act_bits(M, K, seed=11):
    return synth.bits16(synth.to_bf16(synth.activation_f32(seed, M, K, 1.0, 0.01, 20.0)))


@pytest.mark.parametrize("elem", [O.E2M1, O.E4M3])
def test_dequant_requant_is_identity(elem):
    bits = _act_bits(64, 1024)
    codes, scales = O.quantize_mx_bf16(bits, elem)
    deq = O.dequantize_mx(codes, scales, 1024, elem)
    # MX dequantization is exact in BF16 for quantizer output of BF16 input
    deq_bits = _bf16_bits_exact(deq.ravel().tolist()).reshape(deq.shape)
    codes2, scales2 = O.quantize_mx_bf16(deq_bits, elem)
    np.testing.assert_array_equal(scales2, scales)
    np.testing.assert_array_equal(codes2, codes)


def test_nvfp4_dequant_requant_identity_unit_scale():
    bits = _act_bits(32, 256, seed=13)
    codes, scales = O.quantize_nv_bf16(bits, 1.0)
    deq = O.dequantize_nv(codes, scales, 1.0, 256)
    deq_bits = _bf16_bits_exact(deq.ravel().tolist()).reshape(deq.shape)
    codes2, scales2 = O.quantize_nv_bf16(deq_bits, 1.0)
    np.testing.assert_array_equal(scales2, scales)
    np.testing.assert_array_equal(codes2, codes)


@pytest.mark.parametrize("j", [-5, -1, 1, 7])
def test_power_of_two_equivariance(j):
    bits = _act_bits(16, 512, seed=17)
    x = O.bf16_values(bits)
    bits_j = _bf16_bits_exact((x * 2.0 ** j).ravel().tolist()).reshape(x.shape)
    c0, s0 = O.quantize_mx_bf16(bits, O.E2M1)
    c1, s1 = O.quantize_mx_bf16(bits_j, O.E2M1)
    np.testing.assert_array_equal(c1, c0)
    np.testing.assert_array_equal(s1.astype(int), s0.astype(int) + j)


def test_scales_are_powers_of_two_and_block_max_is_4_or_6():
    bits = _act_bits(128, 2048, seed=19)
    codes, scales = O.quantize_mx_bf16(bits, O.E2M1)
    assert scales.max() < 255
    mags = _unpack(codes, 2048) & 7
    blk_max = mags.reshape(128, 64, 32).max(axis=2)
    assert set(np.unique(blk_max)) <= {6, 7}


def test_row_sharding_is_bit_identical():
    bits = _act_bits(96, 640, seed=23)
    c, s = O.quantize_mx_bf16(bits, O.E2M1)
    for a, b in ((0, 1), (5, 37), (37, 96)):
        cs, ss = O.quantize_mx_bf16(bits[a:b], O.E2M1)
        np.testing.assert_array_equal(cs, c[a:b])
        np.testing.assert_array_equal(ss, s[a:b])


def test_quantization_error_sanity_band():
    """Not a pin: relative RMS error of MXFP4 on Gaussian data is of the order of the ~11.6 %
    residual error the W4A8 page reports for real weights."""
    bits = synth.bits16(synth.to_bf16(synth.normal_f32(29, (256, 1024), 0.02)))
    x = O.bf16_values(bits)
    codes, scales = O.quantize_mx_bf16(bits, O.E2M1)
    deq = O.dequantize_mx(codes, scales, 1024)
    rel = np.linalg.norm(deq - x) / np.linalg.norm(x)
    assert 0.05 < rel < 0.25


# ---------------------------------------------------------------------------------------------
# storage arithmetic
# ---------------------------------------------------------------------------------------------
def test_storage_matches_model_card():
    g = _golden("storage_wan_a14b.json")
    h, f = g["hidden"], g["ffn"]
    codes, scales = O.quantize_mx_bf16(np.zeros((1, h), dtype=np.uint16))
    per_elem_mx = (codes.nbytes + scales.nbytes) / h
    assert per_elem_mx == 4.25 / 8
    codes_nv, scales_nv = O.quantize_nv_bf16(np.zeros((1, h), dtype=np.uint16), 1.0)
    assert (codes_nv.nbytes + scales_nv.nbytes) / h == 4.5 / 8
    elems = g["blocks"] * (g["attention_linears_per_block"] * h * h +
                           g["ffn_linears_per_block"] * h * f)
    total = elems * per_elem_mx
    assert abs(total - g["stated_bytes"]) / g["stated_bytes"] < 0.01


# ---------------------------------------------------------------------------------------------
# GEMM, epilogues, low-rank
# ---------------------------------------------------------------------------------------------
def _rand_codes(rng, rows, cols, scale_lo=127, scale_hi=128):
    codes = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(scale_lo, scale_hi, size=(rows, cols // 32)).astype(np.uint8)
    return codes, scales


def test_gemm_exact_grid_case_matches_numpy():
    rng = np.random.default_rng(31)
    M, N, K = 9, 13, 256
    ac, as_ = _rand_codes(rng, M, K)
    wc, ws = _rand_codes(rng, N, K)
    a = O.dequantize_mx(ac, as_, K)
    w = O.dequantize_mx(wc, ws, K)
    # values on the E2M1 grid, unit scales: every partial sum is a multiple of 1/4 below 2^20
    y, t = O.gemm(a, w)
    np.testing.assert_array_equal(y, a @ w.T)
    np.testing.assert_array_equal(t, np.abs(a) @ np.abs(w).T)


def test_gemm_random_scales_and_bias():
    rng = np.random.default_rng(37)
    M, N, K = 7, 11, 320
    ac, as_ = _rand_codes(rng, M, K, 110, 140)
    wc, ws = _rand_codes(rng, N, K, 110, 140)
    bias_bits = synth.bits16(synth.to_f16(synth.normal_f32(5, (N,), 0.01)))
    y, t = O.linear_ref_mx(ac, as_, O.E2M1, wc, ws, K, bias_bits)
    a = O.dequantize_mx(ac, as_, K)
    w = O.dequantize_mx(wc, ws, K)
    b = torch.from_numpy(bias_bits.view(np.int16)).view(torch.float16).to(torch.float64).numpy()
    ref = a @ w.T + b
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-300 + 1e-12 * np.abs(t).max())


def test_gemm_one_hot_weight_and_zero_activation():
    rng = np.random.default_rng(41)
    M, N, K = 5, 8, 64
    ac, as_ = _rand_codes(rng, M, K, 120, 135)
    a = O.dequantize_mx(ac, as_, K)
    w = np.zeros((N, K))
    for n in range(N):
        w[n, 3 * n] = 1.0
    bias = np.arange(N) * 0.125
    y, _ = O.gemm(a, w, bias)
    np.testing.assert_array_equal(y, a[:, 0:3 * N:3] + bias)
    y0, t0 = O.gemm(np.zeros((M, K)), w, bias)
    np.testing.assert_array_equal(y0, np.broadcast_to(bias, (M, N)))
    assert np.all(t0 == 0)


def test_w8a8_reference_exact_and_one_hot():
    """MXFP8 weights (E4M3 codes): with unit scales every product and partial sum is exact in
    fp64, so the reference equals numpy's product of the decoded grids; a one-hot weight (code
    0x38 = 1.0) selects activation columns exactly."""
    rng = np.random.default_rng(43)
    M, N, K = 6, 10, 256
    def e4m3_codes(rows):
        c = rng.integers(0, 256, size=(rows, K), dtype=np.uint8)
        c[(c & 0x7F) == 0x7F] = 0x38  # no NaN codes
        return c
    ac, wc = e4m3_codes(M), e4m3_codes(N)
    as_ = np.full((M, K // 32), 127, dtype=np.uint8)
    ws = np.full((N, K // 32), 127, dtype=np.uint8)
    grid = np.array([O.e4m3_value(c) for c in range(256)])
    a, w = grid[ac], grid[wc]
    y, t = O.linear_ref_mx(ac, as_, O.E4M3, wc, ws, K, None, w_elem=O.E4M3)
    np.testing.assert_array_equal(y, a @ w.T)
    np.testing.assert_array_equal(t, np.abs(a) @ np.abs(w).T)
    oh = np.zeros((N, K), dtype=np.uint8)
    for n in range(N):
        oh[n, 5 * n + 1] = 0x38
    y1, _ = O.linear_ref_mx(ac, as_, O.E4M3, oh, ws, K, None, w_elem=O.E4M3)
    np.testing.assert_array_equal(y1, a[:, 1:5 * N + 1:5])
    # the same bytes read as E2M1 weights give a different matrix: the element type is honoured
    y2, _ = O.linear_ref_mx(ac, as_, O.E4M3, np.ascontiguousarray(oh[:, : K // 2]), ws, K, None)
    assert not np.array_equal(y2, y1)


def test_gelu_matches_torch_and_identities():
    y = np.concatenate([np.linspace(-12, 12, 4001), [0.0, -0.0, 1e-30, -1e-30]])
    g = O.gelu_tanh(y)
    ref = torch.nn.functional.gelu(torch.from_numpy(y), approximate="tanh").numpy()
    # the formula cancels in 1 + tanh(.) for large negative y: compare against |y| there
    assert np.all(np.abs(g - ref) <= 1e-14 * np.abs(ref) + 4e-16 * np.abs(y))
    assert O.gelu_tanh(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(O.gelu_tanh(y) - O.gelu_tanh(-y), y, rtol=1e-13, atol=1e-15)


def test_lowrank_branch():
    M, K, R, N = 6, 96, 32, 40
    x = _act_bits(M, K, seed=43)
    down = synth.bits16(synth.to_bf16(synth.normal_f32(44, (K, R), 0.02)))
    up = synth.bits16(synth.to_bf16(synth.normal_f32(45, (R, N), 0.02)))
    ub, lr, la = O.lowrank(x, down, up)
    s = O.bf16_values(x) @ O.bf16_values(down)
    u = O.bf16_values(ub)
    # u is a BF16 neighbour of the exact sum, within half an ulp (round to nearest)
    _, ex = np.frexp(np.abs(u))
    ulp = np.ldexp(1.0, ex - 8)
    assert np.all(np.abs(u - s) <= 0.5 * ulp + 1e-12 * np.abs(s))
    upv = O.bf16_values(up)
    np.testing.assert_allclose(lr, u @ upv, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(la, np.abs(u) @ np.abs(upv), rtol=1e-12, atol=1e-15)
    _, lr0, _ = O.lowrank(x, np.zeros_like(down), up)
    assert np.all(lr0 == 0)


# ---------------------------------------------------------------------------------------------
# the seeded generator
# ---------------------------------------------------------------------------------------------
def test_generator_is_deterministic_and_normal():
    a = synth.normal_f32(1001, (100000,), 1.0)
    b = synth.normal_f32(1001, (100000,), 1.0)
    c = synth.normal_f32(1002, (100000,), 1.0)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert abs(a.mean()) < 0.02 and abs(a.std() - 1.0) < 0.02
    # prefix property of a counter-based stream
    np.testing.assert_array_equal(synth.normal_f32(1001, (1000,), 1.0), a[:1000])
    idx = synth.outlier_channels(1004, 512, 5)
    assert len(set(idx.tolist())) == 5 and idx.min() >= 0 and idx.max() < 512
    x = synth.activation_f32(1000, 4, 512, 1.0, 0.01, 20.0)
    plain = synth.normal_f32(1001, (4, 512), 1.0)
    ratio = np.abs(x / np.where(plain == 0, 1, plain))
    cols = np.where(np.all(np.isclose(ratio, 20.0), axis=0))[0]
    assert sorted(cols.tolist()) == sorted(idx.tolist())


# ---------------------------------------------------------------------------------------------
# the producer in front of a quantized linear: LayerNorm + modulation
# ---------------------------------------------------------------------------------------------
def _f32(seed, n, sigma, mean=0.0):
    return (synth.normal_f32(seed, (n,), sigma) + np.float32(mean)).astype(np.float32)


def test_norm_modulate_matches_torch_layer_norm():
    """torch's float64 layer_norm is an independent implementation of the normalization."""
    rows, cols = 7, 320
    x_bits = synth.bits16(synth.to_bf16(synth.activation_f32(61, rows, cols, 1.0, 0.02, 30.0)))
    x = O.bf16_values(x_bits)
    g, b = _f32(62, cols, 0.1, 1.0), _f32(63, cols, 0.1)
    for eps in (1e-6, 1e-2):
        ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (cols,), eps=eps).numpy()
        np.testing.assert_allclose(O.norm_modulate(x_bits, eps), ref, rtol=1e-12, atol=1e-12)
        ref_aff = torch.nn.functional.layer_norm(torch.from_numpy(x), (cols,),
                                                 torch.from_numpy(g.astype(np.float64)),
                                                 torch.from_numpy(b.astype(np.float64)), eps).numpy()
        np.testing.assert_allclose(O.norm_modulate(x_bits, eps, gamma=g, beta=b), ref_aff,
                                   rtol=1e-12, atol=1e-12)


def test_norm_modulate_identities():
    rows, cols = 5, 256
    x_bits = synth.bits16(synth.to_bf16(synth.activation_f32(64, rows, cols, 1.0, 0.0, 1.0)))
    s, t = _f32(65, cols, 0.2), _f32(66, cols, 0.3)
    h = O.norm_modulate(x_bits, 0.0)
    # eps = 0: zero mean and unit (biased) variance per row
    np.testing.assert_allclose(h.mean(axis=1), 0.0, atol=1e-14)
    np.testing.assert_allclose((h * h).mean(axis=1), 1.0, rtol=1e-13)
    # eps = 0: invariant under x -> 2x (exact in both BF16 and fp64)
    x2 = O.bf16_rne_array(2.0 * O.bf16_values(x_bits))
    np.testing.assert_array_equal(O.norm_modulate(x2, 0.0), h)
    # modulation is applied after the normalization, per column
    hm = O.norm_modulate(x_bits, 0.0, scale=s, shift=t)
    np.testing.assert_allclose(hm, h * (1.0 + s.astype(np.float64)) + t.astype(np.float64),
                               rtol=1e-15, atol=1e-15)
    # a constant row (exact sums) normalizes to 0, so the output is beta * (1 + scale) + shift
    const = np.full((1, cols), 0x3FC0, dtype=np.uint16)  # 1.5
    b = _f32(67, cols, 0.5)
    hc = O.norm_modulate(const, 1e-6, beta=b, scale=s, shift=t)
    np.testing.assert_array_equal(hc[0], b.astype(np.float64) * (1.0 + s.astype(np.float64))
                                  + t.astype(np.float64))


# ---------------------------------------------------------------------------------------------
# microscaled attention
# ---------------------------------------------------------------------------------------------
def _attn_inputs(BH, S, D, kvb, seed, same_keys=False):
    q = synth.bits16(synth.to_bf16(synth.normal_f32(seed, (BH * S, D), 1.0)))
    kf = synth.normal_f32(seed + 1, (BH * S, D), 1.0)
    if same_keys:
        kf = np.tile(kf[:1], (BH * S, 1))
    k = synth.bits16(synth.to_bf16(kf))
    v = synth.bits16(synth.to_bf16(synth.normal_f32(seed + 2, (BH * S, D), 1.0)))
    qc, qs = O.quantize_mx_bf16(q, O.E2M1)
    kc, ks = O.quantize_mx_bf16(k, O.E2M1)
    vtc, vts = O.quantize_vt_mx8(v, BH, S, D, kvb)
    return qc, qs, kc, ks, vtc, vts


def _vt_dequant(vtc, vts, BH, S, D):
    Sp = vtc.shape[2]
    vt = O.dequantize_mx(vtc.reshape(BH * D, Sp), vts.reshape(BH * D, Sp // 32), Sp, O.E4M3)
    return vt.reshape(BH, D, Sp)[:, :, :S].transpose(0, 2, 1)  # [BH, S, D]


def test_attention_single_key_and_identical_keys_are_exact():
    BH, D, kvb = 2, 128, 64
    # one key: p = 1 exactly, so out = v^ of that key
    qc, qs, kc, ks, vtc, vts = _attn_inputs(BH, 1, D, kvb, 71)
    out, bnd, _ = O.attention_mx(qc, qs, kc, ks, vtc, vts, BH, 1, D, kvb, D ** -0.5)
    np.testing.assert_array_equal(out, _vt_dequant(vtc, vts, BH, 1, D).reshape(BH, D))
    # identical keys: every s is equal, every p is 1 (quantized exactly), out = mean of v^
    S = 100
    qc, qs, kc, ks, vtc, vts = _attn_inputs(1, S, D, kvb, 72, same_keys=True)
    out, _, _ = O.attention_mx(qc, qs, kc, ks, vtc, vts, 1, S, D, kvb, D ** -0.5, qrows=[0, 57, 99])
    mean = _vt_dequant(vtc, vts, 1, S, D)[0].mean(axis=0)
    np.testing.assert_allclose(out, np.broadcast_to(mean, (3, D)), rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("S,kvb", [(130, 64), (77, 32), (64, 64)])
def test_attention_matches_softmax_attention_within_p_quantization(S, kvb):
    """torch's float64 softmax attention on the dequantized Q, K, V is an independent reference;
    the oracle differs from it only by the E4M3 rounding of p (at most 1/8 of p, saturation at
    the block maximum included), so |out - ref| <= sum_j p_j |v_j| / (8 l)."""
    BH, D = 2, 128
    qc, qs, kc, ks, vtc, vts = _attn_inputs(BH, S, D, kvb, 73 + S)
    out, bnd, ab = O.attention_mx(qc, qs, kc, ks, vtc, vts, BH, S, D, kvb, D ** -0.5)
    qd = O.dequantize_mx(qc, qs, D).reshape(BH, S, D)
    kd = O.dequantize_mx(kc, ks, D).reshape(BH, S, D)
    vd = _vt_dequant(vtc, vts, BH, S, D)
    sc = torch.from_numpy(qd) @ torch.from_numpy(kd).transpose(1, 2) * D ** -0.5
    p = torch.softmax(sc, dim=-1)
    ref = (p @ torch.from_numpy(np.ascontiguousarray(vd))).numpy().reshape(BH * S, D)
    tol = (p @ torch.from_numpy(np.abs(np.ascontiguousarray(vd)))).numpy().reshape(BH * S, D) / 8 + 1e-12
    assert np.all(np.abs(out - ref) <= tol)
    assert np.all(bnd >= 0) and np.all(ab > 0)
    # the oracle's own p-rounding bound also covers the distance to the unquantized attention
    assert np.all(np.abs(out - ref) <= 4 * bnd + 1e-12)


def test_vt_quantizer_pads_and_round_trips():
    BH, S, D, kvb = 2, 70, 128, 64
    v = synth.bits16(synth.to_bf16(synth.normal_f32(79, (BH * S, D), 1.0)))
    vtc, vts = O.quantize_vt_mx8(v, BH, S, D, kvb)
    assert vtc.shape == (BH, D, 128) and vts.shape == (BH, D, 4)
    assert np.all(vtc[:, :, S:] == 0) and np.all(vts[:, :, 3] == 0)  # keys 96..127 are all padding
    vd = _vt_dequant(vtc, vts, BH, S, D)
    x = O.bf16_values(v).reshape(BH, S, D)
    # per element: half an E4M3 step (1/16 relative), 1/8 at a saturated block maximum, and half
    # the subnormal quantum 2^(e - 9) of its 32-key block
    e = np.repeat(vts.astype(np.float64) - 127, 32, axis=2)[:, :, :S].transpose(0, 2, 1)
    assert np.all(np.abs(vd - x) <= np.abs(x) / 8 + 2.0 ** (e - 10))


def _cross_inputs(BH, Sq, Skv, D, kvb, seed):
    q = synth.bits16(synth.to_bf16(synth.normal_f32(seed, (BH * Sq, D), 1.0)))
    k = synth.bits16(synth.to_bf16(synth.normal_f32(seed + 1, (BH * Skv, D), 1.0)))
    v = synth.bits16(synth.to_bf16(synth.normal_f32(seed + 2, (BH * Skv, D), 1.0)))
    qc, qs = O.quantize_mx_bf16(q, O.E2M1)
    kc, ks = O.quantize_mx_bf16(k, O.E2M1)
    vtc, vts = O.quantize_vt_mx8(v, BH, Skv, D, kvb)
    return qc, qs, kc, ks, vtc, vts


def test_cross_attention_single_key_is_exact():
    """Queries and keys of different lengths: with one key every query's output is that key's v^."""
    BH, Sq, D, kvb = 2, 5, 128, 64
    qc, qs, kc, ks, vtc, vts = _cross_inputs(BH, Sq, 1, D, kvb, 81)
    out, _, _ = O.attention_mx(qc, qs, kc, ks, vtc, vts, BH, Sq, D, kvb, D ** -0.5, S_kv=1)
    vhat = _vt_dequant(vtc, vts, BH, 1, D).reshape(BH, 1, D)
    np.testing.assert_array_equal(out.reshape(BH, Sq, D), np.broadcast_to(vhat, (BH, Sq, D)))


@pytest.mark.parametrize("Sq,Skv,kvb", [(40, 130, 64), (130, 40, 64), (7, 77, 32)])
def test_cross_attention_matches_softmax_attention_within_p_quantization(Sq, Skv, kvb):
    """As the self-attention pin, with Sq query rows and Skv key / value rows per head."""
    BH, D = 2, 128
    qc, qs, kc, ks, vtc, vts = _cross_inputs(BH, Sq, Skv, D, kvb, 90 + Sq + Skv)
    out, bnd, ab = O.attention_mx(qc, qs, kc, ks, vtc, vts, BH, Sq, D, kvb, D ** -0.5, S_kv=Skv)
    qd = O.dequantize_mx(qc, qs, D).reshape(BH, Sq, D)
    kd = O.dequantize_mx(kc, ks, D).reshape(BH, Skv, D)
    vd = _vt_dequant(vtc, vts, BH, Skv, D)
    sc = torch.from_numpy(qd) @ torch.from_numpy(kd).transpose(1, 2) * D ** -0.5
    p = torch.softmax(sc, dim=-1)
    ref = (p @ torch.from_numpy(np.ascontiguousarray(vd))).numpy().reshape(BH * Sq, D)
    tol = (p @ torch.from_numpy(np.abs(np.ascontiguousarray(vd)))).numpy().reshape(BH * Sq, D) / 8 + 1e-12
    assert np.all(np.abs(out - ref) <= tol)
    assert np.all(np.abs(out - ref) <= 4 * bnd + 1e-12)


# ---------------------------------------------------------------------------------------------
# NVFP4 decode with a global scale other than 1 (NVFP4 model card, Model Details: one FP32
# global scale per tensor; value = code * block scale * global scale, decode direction)
# ---------------------------------------------------------------------------------------------
_E4M3_ALL_F = [None if (b & 0x7F) == 0x7F else
               Fraction(float(torch.tensor([b], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)[0]))
               for b in range(256)]


def _e2m1_f(code):
    """E2M1 code -> Fraction, from the golden grid (sign bit 3)."""
    v = _E2M1_F[code & 7]
    return -v if code & 8 else v


@pytest.mark.parametrize("sg", [40.0 / 2688.0, 3.0 / 7.0, 1e-3])
def test_nvfp4_dequantize_is_exact_product_with_global_scale(sg):
    """dequantize_nv(quantize_nv(x, sg), sg) is code * sb * sg as an exact rational (the three
    factors carry 2, 4 and 24 significant bits, so fp64 holds the product exactly).  Reading the
    global scale the other way (/sg) or dropping it fails."""
    sg32 = float(np.float32(sg))
    bits = _blocks_for_nv(48, 101)
    codes, scales = O.quantize_nv_bf16(bits, sg32)
    deq = O.dequantize_nv(codes, scales, sg32, 16)
    cod = _unpack(codes, 16)
    g = Fraction(sg32)
    for r in range(bits.shape[0]):
        sb = _E4M3_ALL_F[int(scales[r, 0])]
        for i in range(16):
            assert Fraction(float(deq[r, i])) == _e2m1_f(int(cod[r, i])) * sb * g, (r, i)
    # the quantizer fits that decode: where the block scale amax / (6 sg) is a normal,
    # unsaturated E4M3 value, the block maximum decodes within the E4M3 half step (1/16) of
    # amax, code 6 times sb times sg
    x = O.bf16_values(bits)
    amax = np.abs(x).max(axis=1)
    dmax = np.abs(deq).max(axis=1)
    ratio = amax / (6.0 * sg32)
    ok = (ratio >= 2.0 ** -6) & (ratio <= 448.0)
    assert ok.sum() >= 3
    assert np.all(np.abs(dmax[ok] - amax[ok]) <= amax[ok] / 16 * (1 + 1e-12))


def test_nvfp4_gemm_matches_rational_bruteforce():
    """A 3 x 5 x 64 NVFP4 linear with activation and weight global scales other than 1 and an
    FP16 bias, against exact rational arithmetic on the decoded operands."""
    M, N, K = 3, 5, 64
    sg_a, sg_w = float(np.float32(40.0 / 2688.0)), float(np.float32(0.0123))
    a_bits = synth.bits16(synth.to_bf16(synth.activation_f32(111, M, K, 1.0, 0.05, 30.0)))
    w_bits = synth.bits16(synth.to_bf16(synth.normal_f32(112, (N, K), 0.01)))
    b_bits = synth.bits16(synth.to_f16(synth.normal_f32(113, (N,), 0.01)))
    ac, as_ = O.quantize_nv_bf16(a_bits, sg_a)
    wc, ws = O.quantize_nv_bf16(w_bits, sg_w)
    y, t = O.linear_ref_nv(ac, as_, sg_a, wc, ws, sg_w, K, b_bits)
    acod, wcod = _unpack(ac, K), _unpack(wc, K)
    bias = torch.from_numpy(b_bits.view(np.int16)).view(torch.float16).to(torch.float64).numpy()
    for m in range(M):
        for n in range(N):
            s = Fraction(0)
            sa = Fraction(0)
            for k in range(K):
                av = _e2m1_f(int(acod[m, k])) * _E4M3_ALL_F[int(as_[m, k // 16])] * Fraction(sg_a)
                wv = _e2m1_f(int(wcod[n, k])) * _E4M3_ALL_F[int(ws[n, k // 16])] * Fraction(sg_w)
                s += av * wv
                sa += abs(av * wv)
            exact = s + Fraction(float(bias[n]))
            # fp64 summation of K products: within K ulps of the absolute sum
            assert abs(Fraction(float(y[m, n])) - exact) <= Fraction(K * 2.0 ** -52) * (sa + abs(Fraction(float(bias[n]))))
            assert abs(Fraction(float(t[m, n])) - sa) <= Fraction(K * 2.0 ** -52) * sa
    assert np.any(t > 0)


def test_absmax_matches_numpy():
    """mxr_absmax_bf16 against numpy's max of |x| on torch's BF16 decoding, with negative,
    subnormal and extreme values."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((37, 129)).astype(np.float32)
    x[3, 5] = -3.0e38
    x[7, 9] = 1e-40  # BF16 subnormal
    bits = synth.bits16(synth.to_bf16(x))
    ref = float(np.abs(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()).max())
    assert O.absmax_bf16(bits) == ref
    sub = bits[:, 60:]  # without the large negative value
    ref2 = float(np.abs(torch.from_numpy(np.ascontiguousarray(sub).view(np.int16)).view(torch.bfloat16)
                        .to(torch.float64).numpy()).max())
    assert O.absmax_bf16(np.ascontiguousarray(sub)) == ref2
    # the maximum at each corner of the matrix (first / last row and column)
    for r, c in ((0, 0), (0, 128), (36, 0), (36, 128)):
        xc = np.ascontiguousarray(bits[:, 60:].copy())
        xc[r % xc.shape[0], c % xc.shape[1]] = 0xC700  # -32768
        assert O.absmax_bf16(xc) == 32768.0, (r, c)
    assert O.absmax_bf16(np.zeros((2, 3), dtype=np.uint16)) == 0.0
    assert O.absmax_bf16(np.full((1, 4), 0x8001, dtype=np.uint16)) == 2.0 ** -133  # -min subnormal


# ---------------------------------------------------------------------------------------------
# microscaled attention: the probabilities' MXFP8 quantization, seen through a constructed case
# ---------------------------------------------------------------------------------------------
def _encode_exact(v):
    """(E2M1 code, E8M0 byte) whose decoded value is exactly v, by search over the grid."""
    fv = Fraction(v)
    for sb in range(0, 255):
        sc = Fraction(2) ** (sb - 127)
        for c in range(16):
            if _e2m1_f(c) * sc == fv and (c != 8 or v == 0):
                return c, sb
    raise AssertionError(f"{v} is not an E2M1 value times a power of two")


_SINGLE = sorted({sg * m * 2.0 ** e for sg in (1, -1) for m in (1, 3) for e in range(-6, 7)} | {0.0})


def _split3(v):
    """v as a sum of at most three values each exactly an E2M1 value times a power of two."""
    import itertools
    for n in (1, 2, 3):
        for t in itertools.combinations_with_replacement(_SINGLE, n):
            if sum(Fraction(x) for x in t) == Fraction(v):
                return list(t) + [0.0] * (3 - n)
    raise AssertionError(v)


# scores (softmax_scale = ln 2, so c = softmax_scale * log2(e) = 1 and s = q . k) of 128 key
# slots in two blocks of 64: group 0 holds the block maximum 0; group 1 sits 2^20 below it;
# block 1 raises the running maximum to 2; keys 120..127 are past S_kv (masked).
_ATT_S = np.full(128, -48.0)
_ATT_S[[0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11]] = [0, -0.5, -1.5, -3, -8, -16, -17, -18, -24, -0.75, -0.25, -19]
_ATT_S[[32, 33, 34, 35, 36, 37]] = [-20, -20.5, -24, -36, -38, -21.5]
_ATT_S[[64, 65, 66, 67, 96, 97, 98]] = [2, 1, -12, -0.5, -3, -4, -6]
_ATT_SKV = 120


def _attn_constructed():
    D, Skv = 128, _ATT_SKV
    qc = np.zeros((1, D // 2), dtype=np.uint8)
    qs = np.full((1, D // 32), 127, dtype=np.uint8)
    qc[0, [0, 16, 32]] = 2             # q[0] = q[32] = q[64] = 1.0 (E2M1 code 2), others 0
    kc = np.zeros((Skv, D // 2), dtype=np.uint8)
    ks = np.full((Skv, D // 32), 127, dtype=np.uint8)
    for j in range(Skv):
        # k_j[0] + k_j[32] + k_j[64] = s_j, each term in its own 32-element scale block
        for b, t in enumerate(_split3(float(_ATT_S[j]))):
            c, sb = _encode_exact(t)
            kc[j, 16 * b] = c
            ks[j, b] = sb
    # V one-hot: v^[key j, column d] = 1 for d == j (E4M3 1.0 = 0x38, unit scales)
    Sp = 128
    vtc = np.zeros((1, D, Sp), dtype=np.uint8)
    for d in range(Skv):
        vtc[0, d, d] = 0x38
    vts = np.full((1, D, Sp // 32), 127, dtype=np.uint8)
    return qc, qs, kc, ks, vtc, vts


def _e4m3_torch(x):
    """E4M3 rounding (RNE, subnormals kept) by torch's float8_e4m3fn conversion, from float32."""
    t = torch.tensor(np.asarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_attention_probability_quantization_constructed():
    """out * l exposes the quantized probabilities p^ key by key: they must equal an independent
    per-32-key MXFP8 quantization (E8M0 exponent floor(log2 max p) - 8 per group, torch's E4M3
    rounding), o / l must divide by the unquantized l = sum p, absacc must be sum p^ |v^| / l
    exactly, and the flip bound must cover one E4M3 step of p^ without exceeding p / 4 plus the
    group's subnormal quantum.  A scale taken per 64 keys instead of per 32 zeroes group 1 (its
    probabilities lie 2^20 below the block maximum) and fails."""
    D, Skv = 128, _ATT_SKV
    qc, qs, kc, ks, vtc, vts = _attn_constructed()
    out, bnd, ab = O.attention_mx(qc, qs, kc, ks, vtc, vts, 1, 1, D, 64, math.log(2.0), S_kv=Skv)
    out, bnd, ab = out[0], bnd[0], ab[0]
    s = _ATT_S[:Skv]
    # independent evaluation: per block of 64 keys, p = 2^(s - block-running max), quantized per
    # 32-key group; the block-0 terms are rescaled by 2^(m0 - m1) when block 1 raises the max
    m0 = s[:64].max()
    m1 = max(m0, s[64:].max())
    p = np.concatenate([np.exp2(s[:64] - m0), np.exp2(s[64:] - m1)])
    resc = np.concatenate([np.full(64, 2.0 ** (m0 - m1)), np.ones(Skv - 64)])
    p_hat = np.zeros(Skv)
    step_lo = np.zeros(Skv)
    sub_q = np.zeros(Skv)
    for g0 in range(0, Skv, 32):
        grp = slice(g0, min(g0 + 32, Skv))
        _, ex = np.frexp(p[grp].max())
        e = (ex - 1) - 8
        p_hat[grp] = _e4m3_torch(p[grp] * 2.0 ** -e) * 2.0 ** e
        # one E4M3 step at each p^ (normal: 2^(floor(log2 p) - 3); subnormal: 2^(e - 9))
        _, pe = np.frexp(p[grp])
        step_lo[grp] = np.where(p[grp] * 2.0 ** -e >= 2.0 ** -6, np.ldexp(1.0, pe - 1 - 3), 2.0 ** (e - 9))
        sub_q[grp] = 2.0 ** (e - 9)
    l = math.fsum(p * resc)
    ref = p_hat * resc / l
    np.testing.assert_allclose(out[:Skv], ref, rtol=4e-16, atol=0)
    assert np.all(out[Skv:] == 0) and np.all(bnd[Skv:] == 0) and np.all(ab[Skv:] == 0)
    # group 1 is quantized on its own scale: its keys survive (a per-64 scale would zero them)
    assert np.all(out[[32, 33, 34, 35]] > 0) and out[36] == 0.0  # key 36: 2^-10 of its scale, tie to 0
    # keys whose p^ rounds to zero still count in l
    assert out[11] == 0.0 and out[7] == 0.0 and p[11] > 0
    np.testing.assert_array_equal(ab, np.abs(out))
    pos = p > 0
    hi = (p / 4 + sub_q) * resc / l
    lo = step_lo * resc / l
    assert np.all(bnd[:Skv][pos] <= hi[pos] * (1 + 1e-15))
    assert np.all(bnd[:Skv][pos] >= lo[pos] * (1 - 1e-15))


# ---------------------------------------------------------------------------------------------
# storage decoders, the MX dequantizer and the fp32 / fp64 quantizer entry points
# ---------------------------------------------------------------------------------------------
def test_bf16_and_f16_decoders_match_torch_on_every_pattern():
    """mxr_bf16_value and mxr_f16_value on all 65536 patterns against torch's conversions."""
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    tb = torch.from_numpy(allb.view(np.int16))
    ref_b = tb.view(torch.bfloat16).to(torch.float64).numpy()
    ref_h = tb.view(torch.float16).to(torch.float64).numpy()
    got_b = np.array([O.bf16_value(int(b)) for b in allb])
    got_h = O.f16_values(allb)
    for got, ref in ((got_b, ref_b), (got_h, ref_h)):
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan)
        np.testing.assert_array_equal(got[~nan], ref[~nan])
        np.testing.assert_array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    # the vectorised decoder used by the tests agrees with the C one
    with np.errstate(invalid="ignore"):  # signalling NaN patterns
        vec = O.bf16_values(allb)
    np.testing.assert_array_equal(np.isnan(vec), np.isnan(ref_b))
    np.testing.assert_array_equal(vec[~np.isnan(ref_b)], ref_b[~np.isnan(ref_b)])


@pytest.mark.parametrize("elem", [O.E2M1, O.E4M3])
def test_dequantize_mx_is_code_times_power_of_two(elem):
    """mxr_dequantize_mx: value(code) * 2^(byte - 127), NaN for byte 0xFF, from the golden E2M1
    grid / torch's E4M3 decoding (nibble 2j low, 2j + 1 high)."""
    rng = np.random.default_rng(5)
    rows, cols = 9, 256
    scales = rng.integers(0, 255, size=(rows, cols // 32)).astype(np.uint8)
    scales[3, 2] = 0xFF
    if elem == O.E2M1:
        codes = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
        c = _unpack(codes, cols)
        grid = np.concatenate([E2M1_GRID, -E2M1_GRID])
        val = grid[c]
    else:
        codes = rng.integers(0, 256, size=(rows, cols), dtype=np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x40
        val = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ref = val * np.ldexp(1.0, np.repeat(scales.astype(np.int64) - 127, 32, axis=1))
    ref[np.repeat(scales == 0xFF, 32, axis=1)] = np.nan
    got = O.dequantize_mx(codes, scales, cols, elem)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    np.testing.assert_array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def _mx_blocks_brute(x, emax, grid, sign_shift):
    """Independent MX quantization of [rows, cols] fp64 values: per 32 columns, exponent from
    frexp of the block maximum, argmin-distance grid search with ties to the even index."""
    rows, cols = x.shape
    xb = x.reshape(rows, cols // 32, 32)
    amax = np.abs(xb).max(axis=2, keepdims=True)
    _, ex = np.frexp(amax)
    e = np.clip(np.where(amax == 0, -127, ex - 1 - emax), -127, 127)
    q = np.ldexp(np.abs(xb), -e).reshape(-1)
    idx = _nearest_even(q, grid).reshape(xb.shape)
    codes = idx | (np.signbit(xb).astype(np.int64) << sign_shift)
    return codes.reshape(rows, cols).astype(np.uint8), (e[..., 0] + 127).astype(np.uint8)


@pytest.mark.parametrize("elem", [O.E2M1, O.E4M3])
def test_quantize_mx_f32_and_f64_entry_points(elem):
    """mxr_quantize_mx_f32 (the re-quantization of an fp32 intermediate) and mxr_quantize_mx_f64
    on values that are not BF16-representable, against the independent block brute force; on
    BF16-representable values all three entry points agree."""
    rng = np.random.default_rng(9)
    x32 = (rng.standard_normal((12, 128)) * np.exp(rng.uniform(-6, 6, (12, 1)))).astype(np.float32)
    x32[2, :32] = 0.0
    x32[4, 40] = -0.0
    emax, grid, sh = (2, E2M1_GRID, 3) if elem == O.E2M1 else (8, E4M3_GRID, 7)
    ref_c, ref_s = _mx_blocks_brute(x32.astype(np.float64), emax, grid, sh)
    for fn, arg in ((O.quantize_mx_f32, x32), (O.quantize_mx_f64, x32.astype(np.float64))):
        c, s = fn(arg, elem)
        np.testing.assert_array_equal(s, ref_s)
        np.testing.assert_array_equal(_unpack(c, 128) if elem == O.E2M1 else c, ref_c)
    bits = synth.bits16(synth.to_bf16(x32))
    cb, sb = O.quantize_mx_bf16(bits, elem)
    c32, s32 = O.quantize_mx_f32(O.bf16_values(bits).astype(np.float32), elem)
    np.testing.assert_array_equal(cb, c32)
    np.testing.assert_array_equal(sb, s32)


def test_bf16_rne_array_matches_torch():
    rng = np.random.default_rng(3)
    f = np.concatenate([rng.standard_normal(4000), rng.standard_normal(200) * 1e-39]).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(O.bf16_rne_array(f.astype(np.float64)), ref)
