"""The linear layer driven from a C program through include/mxfp.h (tests/c/linear_from_c.c,
built with the C compiler): its FP32 output against the oracle, within the GEMM tolerance."""
import os
import subprocess

import numpy as np
import pytest

import oracle as O
from fp4_block_scaled_amd import synth
from _util import activation_bits, assert_within, f16_bits, weight_bits
from test_abi import _build_c_caller

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,N", [(256, 512, 512), (300, 1024, 640), (1000, 2048, 1280)])
def test_linear_from_c_vs_oracle(tmp_path, M, K, N):
    exe = _build_c_caller(str(tmp_path))
    a = activation_bits(M, K, seed_base=18000 + M)
    w = weight_bits(N, K, seed=18100 + N)
    b = f16_bits(synth.normal_f32(18200 + N, (N,), 0.01))
    paths = {n: str(tmp_path / f"{n}.bin") for n in ("a", "w", "b", "y")}
    a.astype("<u2").tofile(paths["a"])
    w.astype("<u2").tofile(paths["w"])
    b.astype("<u2").tofile(paths["b"])
    r = subprocess.run([exe, paths["a"], paths["w"], paths["b"], paths["y"], str(M), str(K), str(N)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    y = np.fromfile(paths["y"], dtype="<f4").reshape(M, N)
    ac, as_ = O.quantize_mx_bf16(a, O.E2M1)
    wc, ws = O.quantize_mx_bf16(w, O.E2M1)
    y_ref, abs_sum = O.linear_ref_mx(ac, as_, O.E2M1, wc, ws, K, b)
    assert_within(y, y_ref, abs_sum, what="linear from C")
