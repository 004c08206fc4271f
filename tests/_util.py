"""Shared helpers of the test-suite: inputs, tolerances, comparisons."""
import numpy as np
import torch

import oracle as O
from fp4_block_scaled_amd import synth

# fp32 output rounding allowance on top of the GEMM tolerance 2e-3 * sum_k |a_k w_k|: the F32
# output itself is the exact sum rounded to binary32 (<= 2^-24 relative), doubled for margin.
F32_ULP = 2.0 ** -23


def unpack_fp4(packed: np.ndarray, n: int) -> np.ndarray:
    out = np.empty(packed.shape[:-1] + (n,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    return synth.bits16(synth.to_bf16(x))


def f16_bits(x: np.ndarray) -> np.ndarray:
    return synth.bits16(synth.to_f16(x))


def to_dev_bf16(bits: np.ndarray, dev="cuda"):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def to_dev_f16(bits: np.ndarray, dev="cuda"):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16).to(dev)


def dev_bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_rne_of_f32(y: np.ndarray) -> np.ndarray:
    """BF16 bit patterns of binary32 values, round to nearest even (torch's conversion)."""
    return synth.bits16(torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32)).to(torch.bfloat16))


def assert_within(y_gpu: np.ndarray, y_ref: np.ndarray, abs_sum: np.ndarray, extra=None,
                  what="GEMM"):
    """|y_gpu - y_ref| <= 2e-3 * sum|a w| (+ extra) + F32 rounding of the result."""
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    tol = 2e-3 * abs_sum + F32_ULP * np.abs(y_ref)
    if extra is not None:
        tol = tol + extra
    bad = err > tol
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} elements outside tolerance; first {idx.tolist()}; "
            f"max err/tol {np.max(err / np.maximum(tol, 1e-300)):.3g}")
    return float(np.max(err / np.maximum(tol, 1e-300)))


def activation_bits(M, K, seed_base=9000, sigma=1.0, frac=0.01, factor=20.0):
    return bf16_bits_from_f32(synth.activation_f32(seed_base, M, K, sigma, frac, factor))


def weight_bits(N, K, seed=9102, sigma=0.02):
    return bf16_bits_from_f32(synth.normal_f32(seed, (N, K), sigma))


def sample_rows(M: int, count: int, seed: int = 5) -> np.ndarray:
    """Seeded sample of row indices that always includes the first rows and the last (ragged
    tail) rows."""
    rng = np.random.default_rng(seed)
    head = np.arange(min(M, 32))
    tail = np.arange(max(0, M - 96), M)
    mid = rng.choice(M, size=min(M, count), replace=False)
    return np.unique(np.concatenate([head, mid, tail]))


def tile_mx(codes: np.ndarray, scales: np.ndarray, rows: int, cols: int, fp8: bool):
    """The tiled GEMM operand layout of include/mxfp.h, built from row-major codes [rows, cols/2]
    (FP4) or [rows, cols] (FP8) and scales [rows, cols/32] by plain index arithmetic: rows padded
    to a multiple of 256 with zeros; 1 KB code tiles of 16 (FP4) or 8 (FP8) rows x 128 columns,
    16-byte pieces XOR-placed by the row; 256-byte scale tiles of 64 rows x 4 bytes."""
    rp = (rows + 255) // 256 * 256
    nkc = cols // 128
    row_bytes = cols if fp8 else cols // 2
    c = np.zeros((rp, row_bytes), dtype=np.uint8)
    c[:rows] = codes.reshape(rows, row_bytes)
    s = np.zeros((rp, cols // 32), dtype=np.uint8)
    s[:rows] = scales.reshape(rows, cols // 32)
    out_c = np.zeros(rp * row_bytes, dtype=np.uint8)
    out_s = np.zeros(rp * (cols // 32), dtype=np.uint8)
    trows, pieces = (8, 8) if fp8 else (16, 4)
    for r in range(rp):
        for kb in range(nkc):
            base = ((r // trows) * nkc + kb) * 1024 + (r % trows) * (1024 // trows)
            for g in range(pieces):
                slot = g ^ (((r >> 1) & 7) if fp8 else ((r >> 2) & 3))
                src = c[r, kb * 16 * pieces + 16 * g: kb * 16 * pieces + 16 * g + 16]
                out_c[base + 16 * slot: base + 16 * slot + 16] = src
            sb = ((r // 64) * nkc + kb) * 256 + (r % 64) * 4
            out_s[sb: sb + 4] = s[r, 4 * kb: 4 * kb + 4]
    return out_c, out_s


def split_exact(v: float, nterms: int = 3):
    """v as a sum of at most `nterms` values each of the form +-2^a or +-1.5 * 2^a (a in
    [-6, 6]): values that MXFP4 holds exactly when each sits alone in its 32-element block
    (an E2M1 code 4 or 6 times a power-of-two scale).  Padded with zeros."""
    import itertools
    from fractions import Fraction
    single = sorted({s * m * 2.0 ** e for s in (1, -1) for m in (1, 1.5) for e in range(-6, 7)})
    for n in range(1, nterms + 1):
        for t in itertools.combinations_with_replacement(single, n):
            if sum(Fraction(x) for x in t) == Fraction(v):
                return list(t) + [0.0] * (nterms - n)
    raise ValueError(f"{v} needs more than {nterms} terms")
