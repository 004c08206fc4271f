"""MI355X-native microscaled-FP4 linear layer: thin Python binding over ``libmxfp.so``.

Every step runs in the library's gfx950 kernels; this module only marshals arguments (torch
supplies device memory and the current HIP stream).  There is no CPU fallback: if the native
library is missing or no GPU is present the calls raise.

The C ABI is declared in ``include/mxfp.h``; the functions here carry the same names:
``quantize``, ``dequantize``, ``absmax``, ``nvfp4_global_scale``, ``relayout``, ``tiled_bytes``,
``linear`` (dynamic
activation quantization + block-scaled GEMM + epilogue), ``linear_noalloc`` (the same with the
library's static workspace), ``linear_q`` (pre-quantized activation) and
``linear_workspace_bytes``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch  # loaded first: its HIP runtime is the one the native library binds to

_HERE = os.path.dirname(os.path.abspath(__file__))
# MXFP_LIB selects another build of the same library (a variant built with compile-time knobs)
LIB_PATH = os.environ.get("MXFP_LIB") or os.path.join(_HERE, "libmxfp.so")

MXFP4, MXFP8, NVFP4 = 0, 1, 2
NOALLOC_SCRATCH_BYTES = 64 << 20  # MX_NOALLOC_SCRATCH_BYTES of include/mxfp.h
ROW_MAJOR, TILED = 0, 1
EPI_BIAS, EPI_BIAS_GELU, EPI_BIAS_GELU_QUANT_MXFP4, EPI_BIAS_GELU_QUANT_MXFP4_TILED = 0, 1, 2, 3
OUT_BF16, OUT_F32 = 0, 1
_GROUP = {MXFP4: 32, MXFP8: 32, NVFP4: 16}
_FMT_NAMES = {"mxfp4": MXFP4, "mxfp8": MXFP8, "nvfp4": NVFP4}
_EPI_NAMES = {"bias": EPI_BIAS, "bias_gelu": EPI_BIAS_GELU,
              "bias_gelu_quant_mxfp4": EPI_BIAS_GELU_QUANT_MXFP4,
              "bias_gelu_quant_mxfp4_tiled": EPI_BIAS_GELU_QUANT_MXFP4_TILED}
_LAYOUT_NAMES = {"row_major": ROW_MAJOR, "tiled": TILED}


class MxError(RuntimeError):
    pass


class _QMatrix(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("global_scale", ctypes.c_float), ("fmt", ctypes.c_int32),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("layout", ctypes.c_int32)]


class _LowRank(ctypes.Structure):
    _fields_ = [("down", ctypes.c_void_p), ("up", ctypes.c_void_p), ("rank", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded native library (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MxError(f"native library {LIB_PATH} is missing: run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.mx_abi_version.restype = ctypes.c_int
        L.mx_status_string.argtypes = [ctypes.c_int]
        L.mx_status_string.restype = ctypes.c_char_p
        L.mx_last_error.restype = ctypes.c_char_p
        L.mx_quantize.argtypes = [P, I64, I64, I64, I32, I32, ctypes.c_float, P, P, P]
        SZ = ctypes.POINTER(ctypes.c_size_t)
        L.mx_tiled_bytes.argtypes = [I64, I64, I32, SZ, SZ]
        L.mx_relayout.argtypes = [ctypes.POINTER(_QMatrix), ctypes.POINTER(_QMatrix), P]
        L.mx_dequantize.argtypes = [ctypes.POINTER(_QMatrix), P, I64, P]
        L.mx_absmax.argtypes = [P, I64, I64, I64, P, P]
        L.mx_nvfp4_global_scale.argtypes = [ctypes.c_float]
        L.mx_nvfp4_global_scale.restype = ctypes.c_float
        L.mx_linear_workspace_bytes.argtypes = [I64, I64, I32, I32]
        L.mx_linear_workspace_bytes.restype = ctypes.c_size_t
        L.mx_linear.argtypes = [P, I64, I64, I64, I32, ctypes.c_float, ctypes.POINTER(_QMatrix), P,
                                ctypes.POINTER(_LowRank), I32, I32, P, I64, P, P, ctypes.c_size_t, P]
        L.mx_linear_q.argtypes = [ctypes.POINTER(_QMatrix), ctypes.POINTER(_QMatrix), P, I32, I32,
                                  P, I64, P, P]
        L.mx_linear_noalloc.argtypes = [P, I64, I64, I64, I32, ctypes.c_float, ctypes.POINTER(_QMatrix),
                                        P, ctypes.POINTER(_LowRank), I32, I32, P, I64, P, P]
        F = ctypes.c_float
        L.mx_norm.argtypes = [P, I64, I64, I64, F, P, P, P, P, P, I64, P]
        L.mx_norm_quantize.argtypes = [P, I64, I64, I64, F, P, P, P, P, I32, I32, P, P, P]
        L.mx_quantize_vt.argtypes = [P, I64, I64, I64, I64, I64, P, P, P]
        L.mx_attention.argtypes = [P, P, I64, I64, P, P, I64, I64, P, P, I64, I64, I64, I64, F, I32, P,
                                   I64, I64, P]
        for f in ("mx_quantize", "mx_dequantize", "mx_absmax", "mx_linear", "mx_linear_q", "mx_linear_noalloc",
                  "mx_tiled_bytes", "mx_relayout", "mx_norm", "mx_norm_quantize",
                  "mx_quantize_vt", "mx_attention"):
            getattr(L, f).restype = ctypes.c_int
        if L.mx_abi_version() != 2:
            raise MxError("libmxfp.so ABI version mismatch")
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        L = lib()
        raise MxError(f"{L.mx_status_string(status).decode()}: {L.mx_last_error().decode()}")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _fmt(fmt) -> int:
    return _FMT_NAMES[fmt] if isinstance(fmt, str) else int(fmt)


def _layout(layout) -> int:
    return _LAYOUT_NAMES[layout] if isinstance(layout, str) else int(layout)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ld(t: torch.Tensor) -> int:
    """Row stride in elements (a single-row tensor may carry any stride for its first dim)."""
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def _need_cuda(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise MxError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise MxError(f"{name} must be {dtype}, got {t.dtype}")


@dataclass
class QMatrix:
    """A quantized matrix: uint8 codes and scales, an NVFP4 global scale (decode direction),
    the format id and the layout.  Row-major: codes [rows, cols/2] (FP4) or [rows, cols] (FP8),
    scales [rows, cols/G].  Tiled (MX formats): flat byte tensors in the GEMM operand layout of
    ``include/mxfp.h``."""
    codes: torch.Tensor
    scales: torch.Tensor
    fmt: int
    rows: int
    cols: int
    global_scale: float = 1.0
    layout: int = ROW_MAJOR

    def _c(self) -> _QMatrix:
        return _QMatrix(self.codes.data_ptr(), self.scales.data_ptr(), self.global_scale,
                        self.fmt, self.rows, self.cols, self.layout)


@dataclass
class LowRank:
    """SVDQuant low-rank branch: down_t BF16 [rank, K] (the K x rank down factor stored
    transposed, K contiguous) and up_t BF16 [N, rank] (the rank x N up factor transposed)."""
    down_t: torch.Tensor
    up_t: torch.Tensor

    @property
    def rank(self) -> int:
        return self.down_t.shape[0]


def tiled_bytes(rows: int, cols: int, fmt="mxfp4"):
    """(code bytes, scale bytes) of a rows x cols matrix in the tiled layout."""
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().mx_tiled_bytes(rows, cols, _fmt(fmt), ctypes.byref(cb), ctypes.byref(sb)))
    return cb.value, sb.value


def empty_qmatrix(rows: int, cols: int, fmt, device="cuda", global_scale: float = 1.0,
                  layout="row_major") -> QMatrix:
    fmt, layout = _fmt(fmt), _layout(layout)
    if layout == TILED:
        cb, sb = tiled_bytes(rows, cols, fmt)
        codes = torch.empty(cb, dtype=torch.uint8, device=device)
        scales = torch.empty(sb, dtype=torch.uint8, device=device)
        return QMatrix(codes, scales, fmt, rows, cols, global_scale, TILED)
    code_cols = cols if fmt == MXFP8 else cols // 2
    codes = torch.empty((rows, code_cols), dtype=torch.uint8, device=device)
    scales = torch.empty((rows, cols // _GROUP[fmt]), dtype=torch.uint8, device=device)
    return QMatrix(codes, scales, fmt, rows, cols, global_scale)


def quantize(x: torch.Tensor, fmt="mxfp4", global_scale: float = 1.0,
             out: Optional[QMatrix] = None, layout="row_major") -> QMatrix:
    """Dynamic quantization of a 2-D BF16 GPU tensor (row stride may exceed its width), into
    the row-major or (MX formats) the tiled layout; ``out`` fixes the layout when given."""
    fmt = _fmt(fmt)
    _need_cuda(x, "x", torch.bfloat16)
    if x.dim() != 2 or x.stride(1) != 1:
        raise MxError("x must be 2-D with unit column stride")
    rows, cols = x.shape
    q = out if out is not None else empty_qmatrix(rows, cols, fmt, x.device, global_scale, layout)
    q.global_scale = global_scale
    _check(lib().mx_quantize(_ptr(x), rows, cols, _ld(x), fmt, q.layout, global_scale,
                             _ptr(q.codes), _ptr(q.scales), _stream()))
    return q


def _vec(v, cols, name):
    if v is None:
        return None
    _need_cuda(v, name, torch.float32)
    if v.dim() != 1 or v.shape[0] != cols or not v.is_contiguous():
        raise MxError(f"{name} must be a contiguous float32 vector of length {cols}")
    return _ptr(v)


def norm(x: torch.Tensor, eps: float = 1e-6, gamma=None, beta=None, scale=None, shift=None,
         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """BF16 h = LayerNorm(x) [* gamma + beta] [* (1 + scale) + shift] (the unfused producer)."""
    _need_cuda(x, "x", torch.bfloat16)
    if x.dim() != 2 or x.stride(1) != 1:
        raise MxError("x must be 2-D with unit column stride")
    rows, cols = x.shape
    y = out if out is not None else torch.empty((rows, cols), dtype=torch.bfloat16, device=x.device)
    _check(lib().mx_norm(_ptr(x), rows, cols, _ld(x), float(eps), _vec(gamma, cols, "gamma"),
                         _vec(beta, cols, "beta"), _vec(scale, cols, "scale"),
                         _vec(shift, cols, "shift"), _ptr(y), _ld(y), _stream()))
    return y


def norm_quantize(x: torch.Tensor, eps: float = 1e-6, gamma=None, beta=None, scale=None, shift=None,
                  fmt="mxfp4", layout="tiled", out: Optional[QMatrix] = None) -> QMatrix:
    """The producer fused with the quantizer: Q(bf16(h)) with h as in norm(), in `layout`."""
    fmt = _fmt(fmt)
    _need_cuda(x, "x", torch.bfloat16)
    if x.dim() != 2 or x.stride(1) != 1:
        raise MxError("x must be 2-D with unit column stride")
    rows, cols = x.shape
    q = out if out is not None else empty_qmatrix(rows, cols, fmt, x.device, 1.0, layout)
    _check(lib().mx_norm_quantize(_ptr(x), rows, cols, _ld(x), float(eps), _vec(gamma, cols, "gamma"),
                                  _vec(beta, cols, "beta"), _vec(scale, cols, "scale"),
                                  _vec(shift, cols, "shift"), fmt, q.layout, _ptr(q.codes),
                                  _ptr(q.scales), _stream()))
    return q


ATTN_HEAD_DIM = 128
ATTN_KVB = 64


def quantize_vt(v: torch.Tensor, out=None):
    """MXFP8 of V transposed along the key axis, the V operand of attention(): v is a 3-D BF16
    [BH, S, D] GPU tensor with unit last stride (any head and row strides, e.g. a transposed view
    of an [S, H, D] projection).  Returns (codes [BH, Sp/64, D, 64] uint8, scales
    [BH, Sp/64, D, 2] uint8): V^T in blocks of 64 keys, Sp = S rounded up to 64 (written into
    ``out`` = (codes, scales) when given)."""
    _need_cuda(v, "v", torch.bfloat16)
    if v.dim() != 3 or v.stride(2) != 1:
        raise MxError("v must be 3-D [BH, S, D] with unit last stride")
    BH, S, D = v.shape
    Sp = (S + ATTN_KVB - 1) // ATTN_KVB * ATTN_KVB
    if out is not None:
        codes, scales = out
        if tuple(codes.shape) != (BH, Sp // 64, D, 64) or tuple(scales.shape) != (BH, Sp // 64, D, 2) or \
                codes.dtype != torch.uint8 or scales.dtype != torch.uint8 or \
                not codes.is_contiguous() or not scales.is_contiguous():
            raise MxError("out must be contiguous uint8 (codes [BH, Sp/64, D, 64], scales [BH, Sp/64, D, 2])")
    else:
        codes = torch.empty((BH, Sp // 64, D, 64), dtype=torch.uint8, device=v.device)
        scales = torch.empty((BH, Sp // 64, D, 2), dtype=torch.uint8, device=v.device)
    _check(lib().mx_quantize_vt(_ptr(v), BH, S, D, v.stride(1), v.stride(0), _ptr(codes), _ptr(scales),
                                _stream()))
    return codes, scales


def attention(q: QMatrix, k: QMatrix, vt, heads: int, softmax_scale: Optional[float] = None,
              layout: str = "bhsd", out_dtype=torch.bfloat16, out: Optional[torch.Tensor] = None):
    """Microscaled attention (head dimension 128): q and k are row-major MXFP4 QMatrix of the
    queries (S_q per head) and keys (S_kv per head, which may differ: cross-attention), and
    vt = quantize_vt(v) of the S_kv values.  layout "bhsd": q/k rows are heads * S rows of 128
    (head-major), out [heads, S_q, 128]; layout "shd": q/k are S x (heads * 128) (one batch of a
    projection), out [S_q, heads * 128].  softmax_scale defaults to 1/sqrt(128)."""
    for t, name in ((q, "q"), (k, "k")):
        if t.fmt != MXFP4 or t.layout != ROW_MAJOR:
            raise MxError(f"{name} must be a row-major MXFP4 QMatrix")
    if q.cols != k.cols:
        raise MxError("q and k widths differ")
    D = ATTN_HEAD_DIM
    if layout == "bhsd":
        if q.cols != D or q.rows % heads or k.rows % heads:
            raise MxError("bhsd: q and k must be (heads * S) x 128")
        Sq, Skv = q.rows // heads, k.rows // heads
        ld_q, hs_q, ld_k, hs_k = D, Sq * D, D, Skv * D
        shape = (heads, Sq, D)
    elif layout == "shd":
        if q.cols != heads * D:
            raise MxError("shd: q and k must be S x (heads * 128)")
        Sq, Skv = q.rows, k.rows
        ld_q = ld_k = heads * D
        hs_q = hs_k = D
        shape = (Sq, heads * D)
    else:
        raise MxError(f"unknown attention layout {layout!r}")
    vc, vs = vt
    nb = (Skv + ATTN_KVB - 1) // ATTN_KVB
    if tuple(vc.shape) != (heads, nb, D, 64) or tuple(vs.shape) != (heads, nb, D, 2):
        raise MxError("vt does not match k's heads and sequence length")
    o = out if out is not None else torch.empty(shape, dtype=out_dtype, device=q.codes.device)
    if tuple(o.shape) != shape or not o.is_contiguous() or o.dtype not in (torch.bfloat16, torch.float32):
        raise MxError(f"out must be a contiguous bfloat16 / float32 tensor of shape {shape}")
    ld_o, hs_o = (D, Sq * D) if layout == "bhsd" else (heads * D, D)
    scale = float(softmax_scale) if softmax_scale is not None else D ** -0.5
    _check(lib().mx_attention(_ptr(q.codes), _ptr(q.scales), ld_q, hs_q, _ptr(k.codes), _ptr(k.scales),
                              ld_k, hs_k, _ptr(vc), _ptr(vs), heads, Sq, Skv, D, scale,
                              1 if o.dtype == torch.float32 else 0, _ptr(o), ld_o, hs_o, _stream()))
    return o


def relayout(q: QMatrix, layout=None) -> QMatrix:
    """A copy of q in the other layout (or the one named): tiled for the GEMM, row-major to
    read it."""
    target = (TILED if q.layout == ROW_MAJOR else ROW_MAJOR) if layout is None else _layout(layout)
    out = empty_qmatrix(q.rows, q.cols, q.fmt, q.codes.device, q.global_scale, target)
    src, dst = q._c(), out._c()
    _check(lib().mx_relayout(ctypes.byref(src), ctypes.byref(dst), _stream()))
    return out


def dequantize(q: QMatrix) -> torch.Tensor:
    y = torch.empty((q.rows, q.cols), dtype=torch.bfloat16, device=q.codes.device)
    qc = q._c()
    _check(lib().mx_dequantize(ctypes.byref(qc), _ptr(y), q.cols, _stream()))
    return y


def absmax(x: torch.Tensor) -> torch.Tensor:
    """Largest |x| of a BF16 GPU matrix, as a one-element float32 GPU tensor."""
    _need_cuda(x, "x", torch.bfloat16)
    out = torch.empty(1, dtype=torch.float32, device=x.device)
    rows, cols = x.shape
    _check(lib().mx_absmax(_ptr(x), rows, cols, _ld(x), _ptr(out), _stream()))
    return out


def nvfp4_global_scale(amax: float) -> float:
    return float(lib().mx_nvfp4_global_scale(float(amax)))


def quantize_weight_nvfp4(w: torch.Tensor) -> QMatrix:
    """NVFP4 weight preparation: the tensor's global scale from its absmax, then quantization."""
    sg = nvfp4_global_scale(absmax(w).item())
    return quantize(w, NVFP4, sg)


def linear_workspace_bytes(M: int, K: int, act_fmt="mxfp4", rank: int = 0) -> int:
    return int(lib().mx_linear_workspace_bytes(M, K, _fmt(act_fmt), rank))


def _epi(e) -> int:
    return _EPI_NAMES[e] if isinstance(e, str) else int(e)


def _alloc_out(M: int, N: int, epi: int, out_dtype, device):
    if epi == EPI_BIAS_GELU_QUANT_MXFP4:
        return empty_qmatrix(M, N, MXFP4, device)
    if epi == EPI_BIAS_GELU_QUANT_MXFP4_TILED:
        return empty_qmatrix(M, N, MXFP4, device, layout=TILED)
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise MxError(f"out_dtype must be torch.bfloat16 or torch.float32, got {out_dtype}")
    return torch.empty((M, N), dtype=out_dtype, device=device)


def _check_out(out, M: int, N: int, epi: int):
    """Shape, dtype and layout of a caller-supplied output (before any launch)."""
    if epi in (EPI_BIAS_GELU_QUANT_MXFP4, EPI_BIAS_GELU_QUANT_MXFP4_TILED):
        if not isinstance(out, QMatrix):
            raise MxError("the re-quantizing epilogues write a QMatrix")
        layout = TILED if epi == EPI_BIAS_GELU_QUANT_MXFP4_TILED else ROW_MAJOR
        if out.fmt != MXFP4 or out.layout != layout or out.rows != M or out.cols != N:
            raise MxError(f"out must be an MXFP4 {M} x {N} QMatrix in the "
                          f"{'tiled' if layout == TILED else 'row-major'} layout")
        for t, name in ((out.codes, "out.codes"), (out.scales, "out.scales")):
            _need_cuda(t, name, torch.uint8)
            if not t.is_contiguous():
                raise MxError(f"{name} must be contiguous")
        if layout == TILED:
            cb, sb = tiled_bytes(M, N, MXFP4)
        else:
            cb, sb = M * (N // 2), M * (N // 32)
        if out.codes.numel() < cb or out.scales.numel() < sb:
            raise MxError(f"out holds {out.codes.numel()} code / {out.scales.numel()} scale bytes, "
                          f"{cb} / {sb} needed")
        return
    if not isinstance(out, torch.Tensor):
        raise MxError("out must be a tensor")
    _need_cuda(out, "out")
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise MxError(f"out must be bfloat16 or float32, got {out.dtype}")
    if out.dim() != 2 or tuple(out.shape) != (M, N) or (M and out.stride(1) != 1) or \
            (M > 1 and out.stride(0) < N):
        raise MxError(f"out must be a {M} x {N} matrix with unit column stride, got "
                      f"{tuple(out.shape)} / strides {tuple(out.stride())}")


def _check_bias(bias, N: int):
    if bias is None:
        return
    _need_cuda(bias, "bias", torch.float16)
    if bias.dim() != 1 or bias.shape[0] != N or not bias.is_contiguous():
        raise MxError(f"bias must be a contiguous float16 vector of length {N}")


def _check_lowrank(lr: LowRank, K: int, N: int):
    d, u = lr.down_t, lr.up_t
    for t, name in ((d, "down_t"), (u, "up_t")):
        _need_cuda(t, f"lowrank.{name}", torch.bfloat16)
        if t.dim() != 2 or not t.is_contiguous():
            raise MxError(f"lowrank.{name} must be a contiguous 2-D tensor")
    r = d.shape[0]
    if tuple(d.shape) != (r, K) or tuple(u.shape) != (N, r):
        raise MxError(f"lowrank factors must be down_t [rank, K={K}] and up_t [N={N}, rank], got "
                      f"{tuple(d.shape)} and {tuple(u.shape)}")


def _out_args(out, epi):
    if epi in (EPI_BIAS_GELU_QUANT_MXFP4, EPI_BIAS_GELU_QUANT_MXFP4_TILED):
        return _ptr(out.codes), out.cols, _ptr(out.scales), OUT_BF16
    od = OUT_F32 if out.dtype == torch.float32 else OUT_BF16
    return _ptr(out), (_ld(out) if out.shape[0] else out.shape[1]), None, od


def linear(a: torch.Tensor, w: QMatrix, bias: Optional[torch.Tensor] = None, act_fmt="mxfp4",
           act_global_scale: float = 1.0, lowrank: Optional[LowRank] = None, epilogue="bias",
           out_dtype=torch.bfloat16, out=None, workspace: Optional[torch.Tensor] = None):
    """y = epilogue(Q(a) . W^T + bias) with a dynamically quantized to ``act_fmt``.

    a: BF16 [M, K] GPU tensor; w: QMatrix [N, K]; bias: FP16 [N] or None.  Returns a BF16/F32
    [M, N] tensor, or a MXFP4 QMatrix [M, N] (row-major or tiled) for the re-quantizing
    epilogues."""
    act_fmt, epi = _fmt(act_fmt), _epi(epilogue)
    _need_cuda(a, "a", torch.bfloat16)
    if a.dim() != 2 or a.stride(1) != 1:
        raise MxError("a must be 2-D with unit column stride")
    M, K = a.shape
    N = w.rows
    _check_bias(bias, N)
    if out is None:
        out = _alloc_out(M, N, epi, out_dtype, a.device)
    _check_out(out, M, N, epi)
    rank = lowrank.rank if lowrank is not None else 0
    if lowrank is not None:
        _check_lowrank(lowrank, K, N)
    need = linear_workspace_bytes(M, K, act_fmt, rank) if M else 0
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=a.device)
    else:
        _need_cuda(workspace, "workspace", torch.uint8)
        if not workspace.is_contiguous():
            raise MxError("workspace must be contiguous")
    wc = w._c()
    lr = None
    if lowrank is not None:
        lr = ctypes.byref(_LowRank(lowrank.down_t.data_ptr(), lowrank.up_t.data_ptr(), rank))
    optr, ld, sptr, od = _out_args(out, epi)
    _check(lib().mx_linear(_ptr(a), M, K, _ld(a) if M else K, act_fmt, act_global_scale, ctypes.byref(wc),
                           _ptr(bias), lr, epi, od, optr, ld, sptr, _ptr(workspace),
                           workspace.numel(), _stream()))
    return out


def linear_noalloc(a: torch.Tensor, w: QMatrix, bias: Optional[torch.Tensor] = None, act_fmt="mxfp4",
                   act_global_scale: float = 1.0, lowrank: Optional[LowRank] = None, epilogue="bias",
                   out_dtype=torch.bfloat16, out=None):
    """linear() through mx_linear_noalloc: the library's static per-GPU workspace instead of a
    caller one (for callers that cannot allocate; pass ``out`` to allocate nothing at all).  The
    workspace must fit NOALLOC_SCRATCH_BYTES; calls that overlap on one GPU race on it."""
    act_fmt, epi = _fmt(act_fmt), _epi(epilogue)
    _need_cuda(a, "a", torch.bfloat16)
    if a.dim() != 2 or a.stride(1) != 1:
        raise MxError("a must be 2-D with unit column stride")
    M, K = a.shape
    N = w.rows
    _check_bias(bias, N)
    if out is None:
        out = _alloc_out(M, N, epi, out_dtype, a.device)
    _check_out(out, M, N, epi)
    rank = lowrank.rank if lowrank is not None else 0
    lr = None
    if lowrank is not None:
        _check_lowrank(lowrank, K, N)
        lr = ctypes.byref(_LowRank(lowrank.down_t.data_ptr(), lowrank.up_t.data_ptr(), rank))
    wc = w._c()
    optr, ld, sptr, od = _out_args(out, epi)
    _check(lib().mx_linear_noalloc(_ptr(a), M, K, _ld(a) if M else K, act_fmt, act_global_scale,
                                   ctypes.byref(wc), _ptr(bias), lr, epi, od, optr, ld, sptr, _stream()))
    return out


def linear_q(a: QMatrix, w: QMatrix, bias: Optional[torch.Tensor] = None, epilogue="bias",
             out_dtype=torch.bfloat16, out=None):
    """The same GEMM and epilogues on a pre-quantized activation QMatrix [M, K]."""
    epi = _epi(epilogue)
    _check_bias(bias, w.rows)
    if out is None:
        out = _alloc_out(a.rows, w.rows, epi, out_dtype, a.codes.device)
    _check_out(out, a.rows, w.rows, epi)
    ac, wc = a._c(), w._c()
    optr, ld, sptr, od = _out_args(out, epi)
    _check(lib().mx_linear_q(ctypes.byref(ac), ctypes.byref(wc), _ptr(bias), epi, od, optr, ld,
                             sptr, _stream()))
    return out
