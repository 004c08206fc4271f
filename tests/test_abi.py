"""The C ABI library: it loads, exports exactly what include/mxfp.h declares, and its host-side
logic (validation, workspace arithmetic, global-scale arithmetic) behaves as documented.  CPU
only: no call here reaches a kernel launch (every one fails validation first or is host-only).
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp.h")


@pytest.fixture(scope="module")
def mx():
    import fp4_block_scaled_amd as m
    return m


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(mx_[a-z0-9_]+)\s*\(", txt)))


def test_header_declares_the_boundary():
    names = _declared()
    for required in ("mx_quantize", "mx_dequantize", "mx_linear", "mx_linear_q", "mx_absmax",
                     "mx_linear_workspace_bytes", "mx_nvfp4_global_scale", "mx_status_string",
                     "mx_last_error", "mx_abi_version"):
        assert required in names


def test_library_exports_every_declared_symbol(mx):
    L = mx.lib()
    for name in _declared():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", mx.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted({l.split()[-1] for l in out.splitlines() if re.search(r" T mx_", l)})
    assert exported == _declared()


def test_status_strings(mx):
    L = mx.lib()
    for code, name in enumerate(["MX_OK", "MX_ERR_NULL", "MX_ERR_SHAPE", "MX_ERR_ALIGN",
                                 "MX_ERR_UNSUPPORTED", "MX_ERR_WORKSPACE", "MX_ERR_HIP"]):
        assert L.mx_status_string(code).decode() == name
    assert L.mx_abi_version() == 2


def test_nvfp4_global_scale_host_arithmetic_matches_oracle(mx):
    for amax in (40.0, 1.0, 0.0078125, 3.140625, 30.0 * 4.5, 1e-30):
        assert mx.nvfp4_global_scale(amax) == O.nv_global_scale(amax)
    assert mx.nvfp4_global_scale(0.0) == 1.0


def test_workspace_bytes(mx):
    ws = mx.linear_workspace_bytes
    r = lambda v: (v + 255) // 256 * 256
    # MX activations with K % 128 == 0 are staged tiled: rows padded to a multiple of 256
    assert ws(75600, 5120, "mxfp4") == r(75776 * 2560) + r(75776 * 160)
    assert ws(4290, 3072, "mxfp8", 32) == r(4352 * 3072) + r(4352 * 96) + r(4290 * 32 * 2)
    assert ws(300, 160, "mxfp4") == r(300 * 80) + r(300 * 5)  # row-major: K % 128 != 0
    assert ws(75600, 5120, "nvfp4") == r(75600 * 2560) + r(75600 * 320)
    assert ws(0, 5120, "mxfp4") == 0


def test_tiled_bytes(mx):
    assert mx.tiled_bytes(75600, 5120, "mxfp4") == (75776 * 2560, 75776 * 160)
    assert mx.tiled_bytes(1, 128, "mxfp8") == (256 * 128, 256 * 4)
    assert mx.tiled_bytes(0, 256, "mxfp4") == (0, 0)
    with pytest.raises(mx.MxError):
        mx.tiled_bytes(16, 160, "mxfp4")   # cols % 128
    with pytest.raises(mx.MxError):
        mx.tiled_bytes(16, 128, "nvfp4")   # MX formats only


FAKE = 0x10000  # an aligned, never dereferenced address


def _rc(st):
    return st


def test_quantize_validation(mx):
    L = mx.lib()
    P = ctypes.c_void_p
    # unknown format
    assert L.mx_quantize(P(FAKE), 4, 64, 64, 7, 0, 1.0, P(FAKE), P(FAKE), None) == 4
    # cols not a multiple of the group
    assert L.mx_quantize(P(FAKE), 4, 48, 48, mx.MXFP4, 0, 1.0, P(FAKE), P(FAKE), None) == 2
    assert L.mx_quantize(P(FAKE), 4, 24, 24, mx.NVFP4, 0, 1.0, P(FAKE), P(FAKE), None) == 2
    # ld < cols
    assert L.mx_quantize(P(FAKE), 4, 64, 32, mx.MXFP4, 0, 1.0, P(FAKE), P(FAKE), None) == 2
    # NVFP4 needs a positive finite global scale
    assert L.mx_quantize(P(FAKE), 4, 64, 64, mx.NVFP4, 0, 0.0, P(FAKE), P(FAKE), None) == 2
    assert L.mx_quantize(P(FAKE), 4, 64, 64, mx.NVFP4, 0, float("inf"), P(FAKE), P(FAKE), None) == 2
    # NULL pointers
    assert L.mx_quantize(None, 4, 64, 64, mx.MXFP4, 0, 1.0, P(FAKE), P(FAKE), None) == 1
    # misaligned input / leading dimension
    assert L.mx_quantize(P(FAKE + 2), 4, 64, 64, mx.MXFP4, 0, 1.0, P(FAKE), P(FAKE), None) == 3
    assert L.mx_quantize(P(FAKE), 4, 64, 68, mx.MXFP4, 0, 1.0, P(FAKE), P(FAKE), None) == 3
    assert "alignment" in L.mx_last_error().decode()
    # tiled layout: MX formats with cols % 128 == 0, 16-byte aligned outputs; unknown layouts
    assert L.mx_quantize(P(FAKE), 4, 96, 96, mx.MXFP4, 1, 1.0, P(FAKE), P(FAKE), None) == 2
    assert L.mx_quantize(P(FAKE), 4, 128, 128, mx.NVFP4, 1, 1.0, P(FAKE), P(FAKE), None) == 4
    assert L.mx_quantize(P(FAKE), 4, 128, 128, mx.MXFP4, 1, 1.0, P(FAKE + 4), P(FAKE), None) == 3
    assert L.mx_quantize(P(FAKE), 4, 128, 128, mx.MXFP4, 5, 1.0, P(FAKE), P(FAKE), None) == 4
    # zero rows is a no-op even with NULL pointers
    assert L.mx_quantize(None, 0, 64, 64, mx.MXFP4, 0, 1.0, None, None, None) == 0


def _qm(mx, rows, cols, fmt, gs=1.0, codes=FAKE, scales=FAKE, layout=0):
    return mx._QMatrix(codes, scales, gs, fmt, rows, cols, layout)


def test_linear_validation(mx):
    L = mx.lib()
    P = ctypes.c_void_p
    byref = ctypes.byref
    w = _qm(mx, 64, 128, mx.MXFP4)

    def call(a=FAKE, M=16, K=128, lda=128, act=mx.MXFP4, ags=1.0, w_=w, bias=None, lr=None,
             epi=0, od=0, out=FAKE, ldo=64, osc=None, ws=FAKE, wsb=1 << 20):
        return L.mx_linear(P(a) if a else None, M, K, lda, act, ags, byref(w_) if w_ else None,
                           P(bias) if bias else None, lr, epi, od, P(out) if out else None, ldo,
                           P(osc) if osc else None, P(ws) if ws else None, wsb, None)

    assert call(w_=None) == 1
    assert call(a=0) == 1
    assert call(out=0) == 1
    assert call(act=mx.NVFP4) == 4                   # NVFP4 activation with an MXFP4 weight
    assert call(w_=_qm(mx, 64, 128, mx.MXFP8)) == 4  # FP8 weights pair with FP8 activations only
    assert call(act=mx.MXFP8, K=160, lda=160, w_=_qm(mx, 64, 160, mx.MXFP8)) == 2  # W8A8 needs K % 128
    assert call(act=mx.MXFP8, M=0, ws=0, w_=_qm(mx, 64, 128, mx.MXFP8)) == 0      # W8A8 accepted
    assert call(K=96) == 2                           # w->cols != K
    assert call(K=100, w_=_qm(mx, 64, 100, mx.MXFP4), lda=104) == 2  # K % 32
    assert call(ldo=32) == 2                         # ld_out < N
    assert call(epi=2) == 1                          # re-quant epilogue without out_scales
    assert call(epi=2, osc=FAKE, w_=_qm(mx, 48, 128, mx.MXFP4), ldo=48) == 2  # N % 32
    assert call(epi=2, osc=FAKE, ldo=128) == 2      # ld_out must be N
    assert call(epi=3, osc=FAKE, act=mx.MXFP8) == 4  # tiled re-quantized output: MXFP4 activations only
    assert call(epi=3, osc=FAKE, w_=_qm(mx, 96, 128, mx.MXFP4), ldo=96) == 2   # N % 128
    assert call(epi=3, osc=FAKE, K=160, lda=160, w_=_qm(mx, 128, 160, mx.MXFP4), ldo=128) == 2  # K % 128
    assert call(epi=3, osc=FAKE + 8, w_=_qm(mx, 128, 128, mx.MXFP4), ldo=128) == 3  # alignment
    assert call(epi=9) == 4
    assert call(od=5) == 4
    assert call(ws=0) == 5
    assert call(wsb=100) == 5
    assert call(ws=FAKE + 16) == 3                   # workspace alignment
    assert call(a=FAKE + 8) == 3
    assert call(bias=FAKE + 2) == 3
    assert call(act=mx.NVFP4, w_=_qm(mx, 64, 128, mx.NVFP4, gs=0.0)) == 2
    assert call(act=mx.NVFP4, ags=-1.0, w_=_qm(mx, 64, 128, mx.NVFP4, gs=1.0)) == 2
    lr_bad = mx._LowRank(FAKE, FAKE, 24)
    assert call(lr=byref(lr_bad)) == 2
    lr_nv = mx._LowRank(FAKE, FAKE, 32)
    assert call(act=mx.NVFP4, w_=_qm(mx, 64, 128, mx.NVFP4), lr=byref(lr_nv)) == 4
    lr_ok = mx._LowRank(FAKE, FAKE, 32)
    big = (1 << 30) // 31 + 8                        # a 32-row block of a would span >= 2 GiB
    assert call(lr=byref(lr_ok), lda=big - big % 8) == 2
    assert call(lr=byref(lr_ok), lda=(1 << 25), M=0, ws=0) == 0  # 31 * 2^25 + 128 < 2^30
    assert call(K=160, lda=160, w_=_qm(mx, 64, 160, mx.MXFP4, layout=1)) == 2  # tiled needs K % 128
    assert call(act=mx.NVFP4, w_=_qm(mx, 64, 128, mx.NVFP4, layout=1)) == 4     # tiled NVFP4
    assert call(w_=_qm(mx, 64, 128, mx.MXFP4, layout=3)) == 4                   # unknown layout
    assert call(M=0, ws=0) == 0                      # empty activation: no-op


def test_linear_noalloc_validation(mx):
    """mx_linear_noalloc checks mx_linear's arguments, then its static workspace limit, before
    any HIP call: an activation whose workspace exceeds MX_NOALLOC_SCRATCH_BYTES is
    MX_ERR_WORKSPACE."""
    L = mx.lib()
    P = ctypes.c_void_p
    byref = ctypes.byref
    K = 5120
    w = _qm(mx, 64, K, mx.MXFP4)

    def call(M, a=FAKE, w_=w, epi=0, ldo=64):
        return L.mx_linear_noalloc(P(a) if a else None, M, K, K, mx.MXFP4, 1.0, byref(w_) if w_ else None,
                                   None, None, epi, 0, P(FAKE), ldo, None, None)

    hdr = open(HEADER).read()
    assert re.search(r"#define MX_NOALLOC_SCRATCH_BYTES \(64u << 20\)", hdr)
    assert mx.NOALLOC_SCRATCH_BYTES == 64 << 20
    assert mx.linear_workspace_bytes(24576, K, "mxfp4") <= mx.NOALLOC_SCRATCH_BYTES
    assert mx.linear_workspace_bytes(24577, K, "mxfp4") > mx.NOALLOC_SCRATCH_BYTES
    assert call(24577) == 5
    assert "static scratch" in L.mx_last_error().decode()
    assert call(10**6) == 5
    assert call(16, w_=None) == 1
    assert call(16, a=0) == 1
    assert call(16, ldo=32) == 2
    assert call(0) == 0  # empty activation: no-op, no device touched


def test_linear_q_validation(mx):
    L = mx.lib()
    P = ctypes.c_void_p
    a = _qm(mx, 16, 128, mx.MXFP4)
    w = _qm(mx, 64, 128, mx.MXFP4)
    assert L.mx_linear_q(None, ctypes.byref(w), None, 0, 0, P(FAKE), 64, None, None) == 1
    a_bad = _qm(mx, 16, 96, mx.MXFP4)
    assert L.mx_linear_q(ctypes.byref(a_bad), ctypes.byref(w), None, 0, 0, P(FAKE), 64, None, None) == 2
    a_mis = _qm(mx, 16, 128, mx.MXFP4, codes=FAKE + 4)
    assert L.mx_linear_q(ctypes.byref(a_mis), ctypes.byref(w), None, 0, 0, P(FAKE), 64, None, None) == 3
    a0 = _qm(mx, 0, 128, mx.MXFP4)
    assert L.mx_linear_q(ctypes.byref(a0), ctypes.byref(w), None, 0, 0, P(FAKE), 64, None, None) == 0


def test_norm_validation(mx):
    L = mx.lib()
    P = ctypes.c_void_p

    def nq(x=FAKE, rows=16, cols=256, ld=256, eps=1e-6, g=None, b=None, sc=None, sh=None, fmt=0,
           layout=1, codes=FAKE, scales=FAKE):
        return L.mx_norm_quantize(P(x) if x else None, rows, cols, ld, eps, P(g) if g else None,
                                  P(b) if b else None, P(sc) if sc else None, P(sh) if sh else None,
                                  fmt, layout, P(codes) if codes else None,
                                  P(scales) if scales else None, None)

    def nn(x=FAKE, rows=16, cols=256, ld=256, eps=1e-6, y=FAKE, ldy=256):
        return L.mx_norm(P(x) if x else None, rows, cols, ld, eps, None, None, None, None,
                         P(y) if y else None, ldy, None)

    assert nq(fmt=2) == 4                        # NVFP4 output is not provided
    assert nq(layout=5) == 4
    assert nq(cols=96, ld=96) == 2               # tiled needs cols % 128
    assert nq(cols=100, ld=104, layout=0) == 2   # cols % 32
    assert nq(cols=7808, ld=7808) == 2           # beyond MX_NORM_MAX_COLS
    assert nq(ld=128) == 2                       # ld_x < cols
    assert nq(eps=0.0) == 2 and nq(eps=float("inf")) == 2
    assert nq(x=0) == 1 and nq(codes=0) == 1 and nq(scales=0) == 1
    assert nq(x=FAKE + 8) == 3 and nq(ld=260) == 3
    assert nq(sc=FAKE + 2) == 3                  # vectors need 4-byte alignment
    assert nq(codes=FAKE + 8) == 3               # tiled codes need 16-byte alignment
    assert nq(rows=0, x=0, codes=0, scales=0) == 0
    assert nn(y=0) == 1
    assert nn(ldy=128) == 2
    assert nn(y=FAKE + 8) == 3
    assert nn(rows=0, x=0, y=0) == 0


def test_attention_validation(mx):
    L = mx.lib()
    P = ctypes.c_void_p

    def vt(v=FAKE, BH=2, S=100, D=128, ld=128, hs=12800, codes=FAKE, scales=FAKE):
        return L.mx_quantize_vt(P(v) if v else None, BH, S, D, ld, hs, P(codes) if codes else None,
                                P(scales) if scales else None, None)

    def at(q=FAKE, k=FAKE, ld=128, hs=12800, v=FAKE, BH=2, S=100, D=128, scale=0.088, dt=0,
           out=FAKE, ldo=128, hso=12800, Skv=None, ldk=None, hsk=None):
        return L.mx_attention(P(q) if q else None, P(FAKE), ld, hs, P(k) if k else None, P(FAKE),
                              ld if ldk is None else ldk, hs if hsk is None else hsk,
                              P(v) if v else None, P(FAKE), BH, S, S if Skv is None else Skv, D, scale, dt,
                              P(out) if out else None, ldo, hso, None)

    assert vt(D=100, ld=104) == 2 and vt(D=0) == 2
    assert vt(BH=70000) == 2 and vt(S=-1) == 2
    assert vt(ld=64) == 3 and vt(hs=12804) == 3
    assert vt(v=0) == 1 and vt(codes=0) == 1
    assert vt(v=FAKE + 8) == 3 and vt(codes=FAKE + 4) == 3
    assert vt(S=0, v=0, codes=0, scales=0) == 0
    assert at(D=64) == 4
    assert at(scale=0.0) == 2 and at(scale=float("nan")) == 2
    assert at(dt=7) == 4
    assert at(ld=192) == 3 and at(hs=64) == 3
    assert at(ldo=100) == 3
    assert at(q=0) == 1 and at(out=0) == 1
    assert at(k=FAKE + 8) == 3 and at(out=FAKE + 8) == 3
    assert at(S=0, q=0, k=0, v=0, out=0) == 0
    assert at(BH=70000) == 2
    assert at(S=1 << 24, ld=512, hs=0) == 2      # K offsets must stay 32-bit
    assert vt(S=(1 << 24) + 1) == 2
    assert at(Skv=0) == 2                        # queries but no keys
    assert at(S=0, Skv=0, q=0, k=0, v=0, out=0) == 0
    assert at(Skv=-1) == 2 and at(Skv=(1 << 24) + 1) == 2
    assert at(ldk=192) == 3 and at(hsk=64) == 3


def test_relayout_validation(mx):
    L = mx.lib()
    rm, ti = _qm(mx, 16, 128, mx.MXFP4), _qm(mx, 16, 128, mx.MXFP4, layout=1)
    assert L.mx_relayout(None, ctypes.byref(ti), None) == 1
    assert L.mx_relayout(ctypes.byref(rm), ctypes.byref(rm), None) == 4        # same layout
    assert L.mx_relayout(ctypes.byref(rm), ctypes.byref(_qm(mx, 8, 128, mx.MXFP4, layout=1)), None) == 2
    assert L.mx_relayout(ctypes.byref(_qm(mx, 16, 96, mx.MXFP4)),
                         ctypes.byref(_qm(mx, 16, 96, mx.MXFP4, layout=1)), None) == 2  # cols % 128
    assert L.mx_relayout(ctypes.byref(_qm(mx, 16, 128, mx.NVFP4)),
                         ctypes.byref(_qm(mx, 16, 128, mx.NVFP4, layout=1)), None) == 4
    assert L.mx_relayout(ctypes.byref(_qm(mx, 16, 128, mx.MXFP4, codes=FAKE + 4)), ctypes.byref(ti), None) == 3
    assert L.mx_relayout(ctypes.byref(_qm(mx, 0, 128, mx.MXFP4)),
                         ctypes.byref(_qm(mx, 0, 128, mx.MXFP4, layout=1)), None) == 0


def test_binding_fails_loudly_without_native_library(mx, monkeypatch, tmp_path):
    monkeypatch.setattr(mx, "_lib", None)
    monkeypatch.setattr(mx, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(mx.MxError):
        mx.lib()


def test_attention_binding_checks_arguments_before_any_call(mx):
    """The binding's shape and format checks run on the host, before the library is called."""
    import torch
    D = mx.ATTN_HEAD_DIM

    def qm(rows, cols, fmt=None, layout=None):
        fmt = mx.MXFP4 if fmt is None else fmt
        return mx.QMatrix(torch.zeros((rows, cols // 2), dtype=torch.uint8),
                          torch.zeros((rows, cols // 32), dtype=torch.uint8), fmt, rows, cols, 1.0,
                          mx.ROW_MAJOR if layout is None else layout)

    def vt(heads, S):
        nb = (S + 63) // 64
        return (torch.zeros((heads, nb, D, 64), dtype=torch.uint8), torch.zeros((heads, nb, D, 2), dtype=torch.uint8))

    q = qm(2 * 100, D)
    with pytest.raises(mx.MxError):
        mx.attention(qm(200, D, fmt=mx.MXFP8), q, vt(2, 100), 2)          # Q must be MXFP4
    with pytest.raises(mx.MxError):
        mx.attention(q, qm(200, D, layout=mx.TILED), vt(2, 100), 2)       # row-major only
    with pytest.raises(mx.MxError):
        mx.attention(q, qm(201, D), vt(2, 100), 2)                        # k rows not heads * S_kv
    with pytest.raises(mx.MxError):
        mx.attention(q, qm(200, 2 * D), vt(2, 100), 2)                    # q and k widths differ
    with pytest.raises(mx.MxError):
        mx.attention(qm(200, 2 * D), qm(200, 2 * D), vt(2, 100), 2)       # bhsd needs 128 columns
    with pytest.raises(mx.MxError):
        mx.attention(q, q, vt(2, 164), 2)                                 # V^T of another length
    with pytest.raises(mx.MxError):
        mx.attention(q, qm(2 * 200, D), vt(2, 100), 2)                    # V^T not of the keys' length
    with pytest.raises(mx.MxError):
        mx.attention(qm(100, 3 * D), qm(100, 3 * D), vt(3, 100), 2, layout="shd")  # heads * 128 columns
    with pytest.raises(mx.MxError):
        mx.attention(q, q, vt(2, 100), 2, layout="sbhd")                  # unknown layout
    with pytest.raises(mx.MxError):
        mx.quantize_vt(torch.zeros((2, 100, D), dtype=torch.bfloat16))    # a host tensor


def test_variant_library_selection():
    """MXFP_LIB points the binding at another build of the library (a compile-time-knob
    variant); unset, it loads the in-tree libmxfp.so.  Variant names are checked before any
    compiler runs."""
    import sys
    code = "import fp4_block_scaled_amd as m; print(m.LIB_PATH)"
    env = dict(os.environ)
    env.pop("MXFP_LIB", None)
    default = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                             text=True, check=True).stdout.strip()
    assert default == os.path.join(ROOT, "fp4_block_scaled_amd", "libmxfp.so")
    env["MXFP_LIB"] = "/nonexistent/libmxfp_variant.so"
    chosen = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                            text=True, check=True).stdout.strip()
    assert chosen == "/nonexistent/libmxfp_variant.so"
    from fp4_block_scaled_amd import build
    with pytest.raises(ValueError):
        build.build_hip(defines=["MX_RING_PP=0"], variant="../escape")


def _build_c_caller(out_dir):
    """Compile tests/c/linear_from_c.c with the C compiler against include/mxfp.h and link it to
    the in-tree library: the header is plain C and the boundary needs no C++ or Python."""
    exe = os.path.join(out_dir, "linear_from_c")
    pkg = os.path.join(ROOT, "fp4_block_scaled_amd")
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-O2", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "linear_from_c.c"), "-o", exe,
           "-L" + pkg, "-lmxfp", "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath," + pkg, "-Wl,-rpath,/opt/rocm/lib"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def test_c_caller_compiles_and_links(tmp_path):
    exe = _build_c_caller(str(tmp_path))
    out = subprocess.run(["nm", "-u", exe], capture_output=True, text=True, check=True).stdout
    for name in ("mx_quantize", "mx_linear", "mx_linear_workspace_bytes", "mx_tiled_bytes",
                 "mx_abi_version", "mx_status_string", "mx_last_error"):
        assert name in out, name
