"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

Only random-number generation lives here (see ``synth.c``): no quantization, rounding or GEMM
arithmetic of the method.  Storage rounding to BF16/FP16 is done by torch's own conversion, which
is IEEE round-to-nearest-even.

Workload recipes: the token counts are the Wan2.2 latent shapes (720p x 81 frames -> 21 x 45 x 80
= 75600 tokens for the A14B experts; 480x832 x 41 frames -> 11 x 15 x 26 = 4290 tokens for
TI2V-5B); the hidden sizes 5120 / 13824 (A14B) and 3072 (TI2V-5B) are those of the quantized
attention and FFN linears listed in the model cards' coverage sections.  Seeds follow
``seed = 1000 * config + tensor``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MXSYNTH_LIB selects another build of synth.c (the sanitizer build)
_LIB_PATH = os.environ.get("MXSYNTH_LIB") or os.path.join(_HERE, "libmxsynth.so")
_lib = None

# tensor ids inside a config's seed space
T_A, T_W, T_BIAS, T_OUTLIER, T_LDOWN, T_LUP, T_W2, T_B2 = 1, 2, 3, 4, 5, 6, 7, 8
T_MSCALE, T_MSHIFT = 9, 10  # modulation vectors of the norm in front of a linear
T_Q, T_K, T_V = 11, 12, 13   # attention inputs


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(_LIB_PATH)
        lib.mxs_normal_f32.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_double,
                                       ctypes.c_void_p]
        lib.mxs_words.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p]
        lib.mxs_outlier_channels.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_void_p, ctypes.c_void_p]
        lib.mxs_scale_columns_f32.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                              ctypes.c_void_p, ctypes.c_int64, ctypes.c_float]
        _lib = lib
    return _lib


def normal_f32(seed: int, shape, sigma: float) -> np.ndarray:
    """fp32(sigma * N(0,1)) drawn from the counter-based stream ``seed``."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    if n:
        _load().mxs_normal_f32(seed, n, float(sigma), out.ctypes.data)
    return out.reshape(shape)


def words(seed: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    if n:
        _load().mxs_words(seed, n, out.ctypes.data)
    return out


def outlier_channels(seed: int, K: int, count: int) -> np.ndarray:
    scratch = np.empty(K, dtype=np.int64)
    out = np.empty(count, dtype=np.int64)
    if count:
        _load().mxs_outlier_channels(seed, K, count, scratch.ctypes.data, out.ctypes.data)
    return out


def activation_f32(seed_base: int, M: int, K: int, sigma: float, outlier_frac: float,
                   outlier_factor: float) -> np.ndarray:
    """N(0, sigma) activations with round(frac*K) outlier channels scaled by ``outlier_factor``
    (applied in fp32, before any storage rounding)."""
    x = normal_f32(seed_base + T_A, (M, K), sigma)
    count = int(round(outlier_frac * K))
    if count and M:
        idx = outlier_channels(seed_base + T_OUTLIER, K, count)
        _load().mxs_scale_columns_f32(x.ctypes.data, M, K, idx.ctypes.data, count,
                                      float(outlier_factor))
    return x


def to_bf16(x_f32: np.ndarray):
    """fp32 -> torch bfloat16 (RNE).  Returns a CPU torch tensor."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x_f32)).to(torch.bfloat16)


def to_f16(x_f32: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x_f32)).to(torch.float16)


def bits16(t) -> np.ndarray:
    """uint16 bit patterns of a 16-bit torch tensor (CPU)."""
    import torch
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@dataclass
class Workload:
    """One linear layer's synthetic operands (shapes and distributions)."""
    name: str
    config: int            # seed space
    M: int
    K: int
    N: int
    fmt: str = "mxfp4"     # weight/activation format: mxfp4 | w4a8 | w8a8 | nvfp4 | norm | attn
    a_sigma: float = 1.0
    outlier_frac: float = 0.01
    outlier_factor: float = 20.0
    w_sigma: float = 0.02
    bias_sigma: float | None = 0.01
    rank: int = 0          # low-rank branch (W4A8 SVDQuant)
    lr_sigma: float = 0.02
    act_amax_static: float | None = None  # NVFP4 static activation calibration amax
    N2: int | None = None  # FFN pair: second linear's N (its K is N)
    extra: dict = field(default_factory=dict)

    @property
    def seed_base(self) -> int:
        return 1000 * self.config

    def activation(self, M: int | None = None) -> np.ndarray:
        return activation_f32(self.seed_base, self.M if M is None else M, self.K, self.a_sigma,
                              self.outlier_frac, self.outlier_factor)

    def weight(self) -> np.ndarray:
        return normal_f32(self.seed_base + T_W, (self.N, self.K), self.w_sigma)

    def bias(self):
        if self.bias_sigma is None:
            return None
        return normal_f32(self.seed_base + T_BIAS, (self.N,), self.bias_sigma)

    def weight2(self) -> np.ndarray:
        return normal_f32(self.seed_base + T_W2, (self.N2, self.N), self.w_sigma)

    def bias2(self):
        return normal_f32(self.seed_base + T_B2, (self.N2,), self.bias_sigma)

    def lora_down(self) -> np.ndarray:
        return normal_f32(self.seed_base + T_LDOWN, (self.K, self.rank), self.lr_sigma)

    def lora_up(self) -> np.ndarray:
        return normal_f32(self.seed_base + T_LUP, (self.rank, self.N), self.lr_sigma)

    def modulation(self):
        """F32 (scale, shift) [K] of the modulation in front of the linear (N(0, 0.1) each)."""
        return (normal_f32(self.seed_base + T_MSCALE, (self.K,), 0.1),
                normal_f32(self.seed_base + T_MSHIFT, (self.K,), 0.1))

    def qkv(self, S: int | None = None):
        """F32 (q, k, v) of self-attention, each S x K (K = heads * head_dim, one batch of the
        projections): N(0, a_sigma); q and k have round(outlier_frac * K) channels scaled by
        outlier_factor (the channel spread of the normalized, rotated queries and keys)."""
        S = self.M if S is None else S
        out = []
        for t in (T_Q, T_K, T_V):
            x = normal_f32(self.seed_base + t, (S, self.K), self.a_sigma)
            count = int(round(self.outlier_frac * self.K)) if t != T_V else 0
            if count and S:
                idx = outlier_channels(self.seed_base + T_OUTLIER + t, self.K, count)
                _load().mxs_scale_columns_f32(x.ctypes.data, S, self.K, idx.ctypes.data, count,
                                              float(self.outlier_factor))
            out.append(x)
        return tuple(out)


WORKLOADS = {
    # smallest MXFP4 W4A4 instance
    "mxfp4_256x512x512": Workload("mxfp4_256x512x512", 1, 256, 512, 512, "mxfp4",
                                  outlier_frac=0.01, outlier_factor=20.0, w_sigma=0.02),
    # Wan2.2-A14B attn1 projection: 21 x 45 x 80 tokens, hidden 5120
    "wan_a14b_attn_75600x5120x5120": Workload(
        "wan_a14b_attn_75600x5120x5120", 2, 75600, 5120, 5120, "mxfp4",
        outlier_frac=0.005, outlier_factor=30.0, w_sigma=0.015),
    # Wan2.2-A14B FFN pair 5120 -> 13824 -> 5120
    "wan_a14b_ffn_75600x5120x13824": Workload(
        "wan_a14b_ffn_75600x5120x13824", 3, 75600, 5120, 13824, "mxfp4",
        outlier_frac=0.005, outlier_factor=30.0, w_sigma=0.01, N2=5120),
    # Wan2.2-TI2V-5B W4A8 SVDQuant, 11 x 15 x 26 tokens, hidden 3072
    "wan_ti2v5b_w4a8_4290x3072x3072": Workload(
        "wan_ti2v5b_w4a8_4290x3072x3072", 4, 4290, 3072, 3072, "w4a8",
        outlier_frac=0.01, outlier_factor=25.0, w_sigma=0.02, bias_sigma=None, rank=32),
    "wan_ti2v5b_w4a8_4290x3072x14336": Workload(
        "wan_ti2v5b_w4a8_4290x3072x14336", 4, 4290, 3072, 14336, "w4a8",
        outlier_frac=0.01, outlier_factor=25.0, w_sigma=0.02, bias_sigma=None, rank=32),
    # MXFP8 W8A8 reference layer at the attention-projection shape; the same seeds (config 2),
    # so the same BF16 operands, as the W4A4 workload
    "wan_a14b_w8a8_75600x5120x5120": Workload(
        "wan_a14b_w8a8_75600x5120x5120", 2, 75600, 5120, 5120, "w8a8",
        outlier_frac=0.005, outlier_factor=30.0, w_sigma=0.015),
    # the LayerNorm + modulation in front of the attention projection, fused with its MXFP4
    # quantizer (same activation seeds as the W4A4 workload; N is unused)
    "wan_a14b_norm_quant_75600x5120": Workload(
        "wan_a14b_norm_quant_75600x5120", 2, 75600, 5120, 5120, "norm",
        outlier_frac=0.005, outlier_factor=30.0),
    # Wan2.2-A14B self-attention at 720p: 75600 tokens, 40 heads of 128 (N unused)
    "wan_a14b_attn_mx_75600x40x128": Workload(
        "wan_a14b_attn_mx_75600x40x128", 6, 75600, 5120, 5120, "attn",
        outlier_frac=0.02, outlier_factor=3.0, extra={"heads": 40}),
    # Wan2.2-TI2V-5B self-attention: 4290 tokens, 24 heads of 128 (N unused)
    "wan_ti2v5b_attn_mx_4290x24x128": Workload(
        "wan_ti2v5b_attn_mx_4290x24x128", 7, 4290, 3072, 3072, "attn",
        outlier_frac=0.02, outlier_factor=3.0, extra={"heads": 24}),
    # NVFP4 at the A14B FFN shape with a static activation global scale (amax 40)
    "wan_a14b_nvfp4_75600x5120x13824": Workload(
        "wan_a14b_nvfp4_75600x5120x13824", 5, 75600, 5120, 13824, "nvfp4",
        outlier_frac=0.005, outlier_factor=30.0, w_sigma=0.01, act_amax_static=40.0),
}
