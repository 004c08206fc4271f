"""CPU oracle for the microscaled-FP4 linear layer and the microscaled attention (ctypes wrapper
over ``mxref.c``).

TEST INFRASTRUCTURE ONLY.  Imported by the tests, by ``__graft_entry__.smoke()`` and by the
benchmark's CPU-baseline leg; never by the product package.  It shares no code with the HIP
path; both consume the same seeded inputs from ``fp4_block_scaled_amd.synth``.

All arrays are numpy; BF16/FP16 values travel as uint16 bit patterns, fp64 values as float64.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MXREF_LIB selects another build of mxref.c (the sanitizer build of oracle/build.py)
LIB_PATH = os.environ.get("MXREF_LIB") or os.path.join(_HERE, "libmxref.so")
E2M1, E4M3 = 0, 1

_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int64


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        L.mxr_bf16_value.argtypes = [ctypes.c_uint16]
        L.mxr_bf16_value.restype = ctypes.c_double
        L.mxr_f16_value.argtypes = [ctypes.c_uint16]
        L.mxr_f16_value.restype = ctypes.c_double
        L.mxr_bf16_rne.argtypes = [ctypes.c_double]
        L.mxr_bf16_rne.restype = ctypes.c_uint16
        for f in ("mxr_e2m1_value", "mxr_e4m3_value", "mxr_e8m0_value"):
            getattr(L, f).argtypes = [ctypes.c_uint]
            getattr(L, f).restype = ctypes.c_double
        L.mxr_e2m1_rne_mag.argtypes = [ctypes.c_double]
        L.mxr_e2m1_rne_mag.restype = ctypes.c_uint
        L.mxr_e4m3_rne_mag.argtypes = [ctypes.c_double]
        L.mxr_e4m3_rne_mag.restype = ctypes.c_uint
        L.mxr_mx_block.argtypes = [_P, ctypes.c_int, ctypes.c_int, _P, _P]
        L.mxr_mx_block.restype = None
        for f in ("mxr_quantize_mx_f64", "mxr_quantize_mx_bf16", "mxr_quantize_mx_f32"):
            getattr(L, f).argtypes = [_P, _I, _I, _I, ctypes.c_int, _P, _P]
            getattr(L, f).restype = ctypes.c_int
        L.mxr_dequantize_mx.argtypes = [_P, _P, _I, _I, ctypes.c_int, _P]
        L.mxr_dequantize_mx.restype = None
        L.mxr_nv_global_scale.argtypes = [ctypes.c_double]
        L.mxr_nv_global_scale.restype = ctypes.c_float
        L.mxr_nv_block.argtypes = [_P, ctypes.c_int, ctypes.c_float, _P, _P]
        L.mxr_nv_block.restype = None
        L.mxr_quantize_nv_bf16.argtypes = [_P, _I, _I, _I, ctypes.c_float, _P, _P]
        L.mxr_quantize_nv_bf16.restype = ctypes.c_int
        L.mxr_dequantize_nv.argtypes = [_P, _P, ctypes.c_float, _I, _I, _P]
        L.mxr_dequantize_nv.restype = None
        L.mxr_gemm_f64.argtypes = [_P, _I, _P, _I, _I, _P, _P, _P]
        L.mxr_gemm_f64.restype = None
        L.mxr_gelu_tanh.argtypes = [ctypes.c_double]
        L.mxr_gelu_tanh.restype = ctypes.c_double
        L.mxr_gelu_tanh_array.argtypes = [_P, _I, _P]
        L.mxr_gelu_tanh_array.restype = None
        L.mxr_lowrank.argtypes = [_P, _I, _I, _I, _P, _I, _P, _I, _P, _P, _P]
        L.mxr_lowrank.restype = None
        L.mxr_bf16_rne_array.argtypes = [_P, _I, _P]
        L.mxr_bf16_rne_array.restype = None
        L.mxr_absmax_bf16.argtypes = [_P, _I, _I, _I]
        L.mxr_absmax_bf16.restype = ctypes.c_double
        L.mxr_norm_modulate.argtypes = [_P, _I, _I, _I, ctypes.c_double, _P, _P, _P, _P, _P]
        L.mxr_norm_modulate.restype = None
        L.mxr_attention_mx.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_int,
                                       ctypes.c_double, _P, _I, _P, _P, _P]
        L.mxr_attention_mx.restype = None
        _lib = L
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


# ---- scalar formats ------------------------------------------------------------------------
def e2m1_value(code: int) -> float:
    return lib().mxr_e2m1_value(code)


def e4m3_value(code: int) -> float:
    return lib().mxr_e4m3_value(code)


def e8m0_value(code: int) -> float:
    return lib().mxr_e8m0_value(code)


def e2m1_rne_mag(q: float) -> int:
    return lib().mxr_e2m1_rne_mag(q)


def e4m3_rne_mag(q: float) -> int:
    return lib().mxr_e4m3_rne_mag(q)


def bf16_value(bits: int) -> float:
    return lib().mxr_bf16_value(bits)


def bf16_rne(v: float) -> int:
    return lib().mxr_bf16_rne(v)


def bf16_rne_array(v: np.ndarray) -> np.ndarray:
    """BF16 bit patterns of exact fp64 values (one rounding each)."""
    v, pv = _c(v, np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().mxr_bf16_rne_array(pv, v.size, out.ctypes.data)
    return out


def f16_values(bits: np.ndarray) -> np.ndarray:
    L = lib()
    return np.array([L.mxr_f16_value(int(b)) for b in np.asarray(bits).ravel()],
                    dtype=np.float64).reshape(np.shape(bits))


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """Exact BF16 -> fp64 (vectorised; the BF16 pattern is the top half of binary32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---- blocks --------------------------------------------------------------------------------
def mx_block(x, elem=E2M1):
    x, px = _c(x, np.float64)
    codes = np.zeros(len(x), dtype=np.uint8)
    scale = np.zeros(1, dtype=np.uint8)
    lib().mxr_mx_block(px, len(x), elem, codes.ctypes.data, scale.ctypes.data)
    return codes, int(scale[0])


def nv_block(x, sg: float):
    x, px = _c(x, np.float64)
    codes = np.zeros(len(x), dtype=np.uint8)
    scale = np.zeros(1, dtype=np.uint8)
    lib().mxr_nv_block(px, len(x), float(sg), codes.ctypes.data, scale.ctypes.data)
    return codes, int(scale[0])


# ---- matrices ------------------------------------------------------------------------------
def _code_cols(cols, elem):
    return cols // 2 if elem == E2M1 else cols


def quantize_mx_bf16(x_bits: np.ndarray, elem=E2M1):
    """Quantize a [rows, cols] BF16 (uint16 bits) matrix; returns (codes, scales)."""
    x, px = _c(x_bits, np.uint16)
    rows, cols = x.shape
    codes = np.empty((rows, _code_cols(cols, elem)), dtype=np.uint8)
    scales = np.empty((rows, cols // 32), dtype=np.uint8)
    rc = lib().mxr_quantize_mx_bf16(px, rows, cols, cols, elem, codes.ctypes.data,
                                    scales.ctypes.data)
    if rc:
        raise ValueError("cols must be a multiple of 32")
    return codes, scales


def quantize_mx_f64(x: np.ndarray, elem=E2M1):
    x, px = _c(x, np.float64)
    rows, cols = x.shape
    codes = np.empty((rows, _code_cols(cols, elem)), dtype=np.uint8)
    scales = np.empty((rows, cols // 32), dtype=np.uint8)
    rc = lib().mxr_quantize_mx_f64(px, rows, cols, cols, elem, codes.ctypes.data,
                                   scales.ctypes.data)
    if rc:
        raise ValueError("cols must be a multiple of 32")
    return codes, scales


def quantize_mx_f32(x: np.ndarray, elem=E2M1):
    x, px = _c(x, np.float32)
    rows, cols = x.shape
    codes = np.empty((rows, _code_cols(cols, elem)), dtype=np.uint8)
    scales = np.empty((rows, cols // 32), dtype=np.uint8)
    rc = lib().mxr_quantize_mx_f32(px, rows, cols, cols, elem, codes.ctypes.data,
                                   scales.ctypes.data)
    if rc:
        raise ValueError("cols must be a multiple of 32")
    return codes, scales


def dequantize_mx(codes, scales, cols: int, elem=E2M1) -> np.ndarray:
    codes, pc = _c(codes, np.uint8)
    scales, ps = _c(scales, np.uint8)
    rows = codes.shape[0]
    out = np.empty((rows, cols), dtype=np.float64)
    lib().mxr_dequantize_mx(pc, ps, rows, cols, elem, out.ctypes.data)
    return out


def nv_global_scale(amax: float) -> float:
    return float(np.float32(lib().mxr_nv_global_scale(float(amax))))


def quantize_nv_bf16(x_bits: np.ndarray, sg: float):
    x, px = _c(x_bits, np.uint16)
    rows, cols = x.shape
    codes = np.empty((rows, cols // 2), dtype=np.uint8)
    scales = np.empty((rows, cols // 16), dtype=np.uint8)
    rc = lib().mxr_quantize_nv_bf16(px, rows, cols, cols, float(sg), codes.ctypes.data,
                                    scales.ctypes.data)
    if rc:
        raise ValueError("cols must be a multiple of 16")
    return codes, scales


def dequantize_nv(codes, scales, sg: float, cols: int) -> np.ndarray:
    codes, pc = _c(codes, np.uint8)
    scales, ps = _c(scales, np.uint8)
    rows = codes.shape[0]
    out = np.empty((rows, cols), dtype=np.float64)
    lib().mxr_dequantize_nv(pc, ps, float(sg), rows, cols, out.ctypes.data)
    return out


def gemm(a: np.ndarray, w: np.ndarray, bias=None):
    """(y, abs_sum): y = a @ w.T + bias summed in fp64, abs_sum = |a| @ |w|.T elementwise."""
    a, pa = _c(a, np.float64)
    w, pw = _c(w, np.float64)
    M, K = a.shape
    N = w.shape[0]
    y = np.empty((M, N), dtype=np.float64)
    t = np.empty((M, N), dtype=np.float64)
    pb = None
    if bias is not None:
        bias, pb = _c(bias, np.float64)
    lib().mxr_gemm_f64(pa, M, pw, N, K, pb, y.ctypes.data, t.ctypes.data)
    return y, t


def gelu_tanh(y: np.ndarray) -> np.ndarray:
    y, py = _c(y, np.float64)
    out = np.empty_like(y)
    lib().mxr_gelu_tanh_array(py, y.size, out.ctypes.data)
    return out


def lowrank(x_bits, down_bits, up_bits):
    """(u_bits [M,R], lr [M,N], lr_abs [M,N]) of the SVDQuant low-rank branch."""
    x, px = _c(x_bits, np.uint16)
    d, pd = _c(down_bits, np.uint16)
    u_, pu = _c(up_bits, np.uint16)
    M, K = x.shape
    R = d.shape[1]
    N = u_.shape[1]
    ub = np.empty((M, R), dtype=np.uint16)
    lr = np.empty((M, N), dtype=np.float64)
    la = np.empty((M, N), dtype=np.float64)
    lib().mxr_lowrank(px, K, M, K, pd, R, pu, N, ub.ctypes.data, lr.ctypes.data, la.ctypes.data)
    return ub, lr, la


def absmax_bf16(x_bits) -> float:
    x, px = _c(x_bits, np.uint16)
    rows, cols = x.shape
    return lib().mxr_absmax_bf16(px, rows, cols, cols)


# ---- composite references -----------------------------------------------------------------
def linear_ref_mx(a_codes, a_scales, a_elem, w_codes, w_scales, K, bias_f16_bits=None, w_elem=E2M1):
    """Reference MX linear on quantized operands: (y, abs_sum) in fp64.  w_elem is E2M1 for the
    MXFP4 weights of W4A4 / W4A8, E4M3 for the MXFP8 weights of the W8A8 reference layer."""
    a = dequantize_mx(a_codes, a_scales, K, a_elem)
    w = dequantize_mx(w_codes, w_scales, K, w_elem)
    bias = None if bias_f16_bits is None else f16_values(bias_f16_bits)
    return gemm(a, w, bias)


def linear_ref_nv(a_codes, a_scales, sg_a, w_codes, w_scales, sg_w, K, bias_f16_bits=None):
    a = dequantize_nv(a_codes, a_scales, sg_a, K)
    w = dequantize_nv(w_codes, w_scales, sg_w, K)
    bias = None if bias_f16_bits is None else f16_values(bias_f16_bits)
    return gemm(a, w, bias)


# ---- the producer of a quantized linear's input --------------------------------------------
def norm_modulate(x_bits, eps: float, gamma=None, beta=None, scale=None, shift=None) -> np.ndarray:
    """fp64 h = LayerNorm(x) [* gamma + beta] [* (1 + scale) + shift] per row (see
    mxr_norm_modulate); the vectors are F32 [cols] or None."""
    x, px = _c(x_bits, np.uint16)
    rows, cols = x.shape
    vecs = []
    for v in (gamma, beta, scale, shift):
        if v is None:
            vecs.append((None, None))
        else:
            a, pa = _c(v, np.float32)
            assert a.shape == (cols,)
            vecs.append((a, pa))
    h = np.empty((rows, cols), dtype=np.float64)
    lib().mxr_norm_modulate(px, rows, cols, cols, float(eps), *[p for _, p in vecs], h.ctypes.data)
    return h


# ---- microscaled attention -------------------------------------------------------------------
def attention_mx(qc, qs, kc, ks, vtc, vts, BH: int, S: int, D: int, kvb: int, softmax_scale: float,
                 qrows=None, S_kv=None):
    """(out, bound, absacc) [nq, D] in fp64 for the listed query rows (all rows if None); see
    mxr_attention_mx.  q codes [BH*S, D/2] + scales [BH*S, D/32]; k codes [BH*S_kv, D/2] + scales;
    V^T codes [BH, D, Sp] E4M3 + scales [BH, D, Sp/32], Sp = S_kv rounded up to kvb.  S_kv
    defaults to S (self-attention)."""
    assert D <= 1024 and kvb <= 256 and kvb % 32 == 0
    Skv = S if S_kv is None else S_kv
    Sp = (Skv + kvb - 1) // kvb * kvb
    arrs = [_c(a, np.uint8) for a in (qc, qs, kc, ks, vtc, vts)]
    assert arrs[2][0].size == BH * Skv * (D // 2) and arrs[4][0].size == BH * D * Sp and arrs[5][0].size == BH * D * (Sp // 32)
    rows = np.arange(BH * S, dtype=np.int64) if qrows is None else np.asarray(qrows, dtype=np.int64)
    rows, pr = _c(rows, np.int64)
    nq = rows.size
    out = np.empty((nq, D)); bnd = np.empty((nq, D)); ab = np.empty((nq, D))
    lib().mxr_attention_mx(*[p for _, p in arrs], BH, S, Skv, D, Sp, kvb, float(softmax_scale), pr, nq,
                           out.ctypes.data, bnd.ctypes.data, ab.ctypes.data)
    return out, bnd, ab


def quantize_vt_mx8(v_bits, BH: int, S: int, D: int, kvb: int):
    """V [BH, S, D] BF16 bits -> (codes [BH, D, Sp], scales [BH, D, Sp/32]): Q_MX8 of V transposed
    along the key axis, keys padded with zeros to Sp = S rounded up to kvb."""
    Sp = (S + kvb - 1) // kvb * kvb
    vt = np.zeros((BH, D, Sp), dtype=np.uint16)
    vt[:, :, :S] = np.asarray(v_bits, dtype=np.uint16).reshape(BH, S, D).transpose(0, 2, 1)
    c, s = quantize_mx_bf16(vt.reshape(BH * D, Sp), E4M3)
    return c.reshape(BH, D, Sp), s.reshape(BH, D, Sp // 32)
