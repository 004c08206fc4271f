// Internal launcher interface between the C ABI (mx_capi.hip) and the kernels (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxk {

// Quantizers / dequantizer / absmax (mx_quant.hip)
hipError_t launch_quant_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int elem,
                           uint8_t* codes, uint8_t* scales, hipStream_t s);
// MX quantization into the tiled GEMM layout (cols % 128 == 0); rows up to the padded count are
// written, the padding with zeros.
hipError_t launch_quant_mx_tiled(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int elem,
                                 uint8_t* codes, uint8_t* scales, hipStream_t s);
// Row-major <-> tiled copy of MX codes and scales (to_tiled: direction).
hipError_t launch_relayout(const uint8_t* src_codes, const uint8_t* src_scales, uint8_t* dst_codes,
                           uint8_t* dst_scales, int64_t rows, int64_t cols, int elem, bool to_tiled,
                           hipStream_t s);
// LayerNorm (+ affine) + modulation of a BF16 [rows, cols] matrix, then: out_kind 0 BF16 y,
// 1 MX codes row-major, 2 MX codes tiled (elem 0 E2M1, 1 E4M3).  cols <= 7680.
hipError_t launch_norm_quant(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, float eps,
                             const float* gamma, const float* beta, const float* scale,
                             const float* shift, int out_kind, int elem, uint16_t* y, int64_t ld_y,
                             uint8_t* codes, uint8_t* scales, hipStream_t s);
hipError_t launch_quant_nv(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, float sg,
                           uint8_t* codes, uint8_t* scales, hipStream_t s);
hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                          int fmt, float sg, uint16_t* y, int64_t ld, hipStream_t s);
hipError_t launch_absmax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, float* out,
                         hipStream_t s);

// GEMMs (mx_gemm.hip)
// EPI_GELU_QUANT_T: the re-quantized output in the tiled layout (rows padded with zeros)
enum { EPI_BIAS = 0, EPI_GELU = 1, EPI_GELU_QUANT = 2, EPI_GELU_QUANT_T = 3 };

struct GemmParams {
  const uint8_t* a_codes;   // [M, K/2] (FP4) or [M, K] (FP8)
  const uint8_t* a_scales;  // [M, K/32] E8M0, or [M, K/16] E4M3 (NVFP4)
  const uint8_t* w_codes;   // [N, K/2] (FP4) or [N, K] (FP8)
  const uint8_t* w_scales;  // [N, K/32] or [N, K/16]
  const uint16_t* bias;     // FP16 [N] or nullptr
  const uint16_t* lr_u;     // BF16 [M, R] or nullptr (low-rank intermediate)
  const uint16_t* lr_up;    // BF16 [N, R]
  void* out;                // BF16 / FP32 [M, ld_out], or FP4 codes [M, N/2]
  uint8_t* out_scales;      // [M, N/32] for the re-quantizing epilogue
  int64_t ld_out;
  float out_scale;          // NVFP4: product of the two global scales, else 1
  int M, N, K, R;
  int epi;
  int out_f32;
  int a_tiled, w_tiled;     // operand layouts: 0 row-major, 1 tiled (MX formats)
};

// act_fp8: activation codes are E4M3 (W4A8); otherwise E2M1.  w_fp8: weight codes are E4M3
// (W8A8, with act_fp8 and K % 128 == 0 only); otherwise E2M1.
hipError_t launch_gemm_mx(const GemmParams& p, bool act_fp8, bool w_fp8, hipStream_t s);
hipError_t launch_gemm_nv(const GemmParams& p, hipStream_t s);
// MXFP4 x MXFP4 linear on a small grid in one launch, from the BF16 activation a (row m at
// a + m * ld_a): quantization and GEMM, output bits equal to launch_quant_mx* + launch_gemm_mx.
// linear_fused_small_ok says when it applies (no low-rank branch, bias/GELU epilogue,
// K % 128 == 0, K <= 896, at most 8 tiles of 256 x 128).
bool linear_fused_small_ok(const GemmParams& p);
hipError_t launch_linear_fused_small(const GemmParams& p, const uint16_t* a, int64_t ld_a, hipStream_t s);
// u[m, r] = bf16_rne(sum_k x[m, k] * down_t[r, k])
hipError_t launch_lowrank_down(const uint16_t* x, int64_t ld_x, const uint16_t* down_t, int M,
                               int K, int R, uint16_t* u, hipStream_t s);
// The same, also quantizing x to MXFP8 in the tiled layout (K % 128 == 0) in the same pass:
// codes and scales of the rows of the 32-row blocks (the tiled padding rows beyond are not written).
hipError_t launch_quant8_lowrank_down(const uint16_t* x, int64_t ld_x, const uint16_t* down_t, int M,
                                      int K, int R, uint16_t* u, uint8_t* codes, uint8_t* scales,
                                      hipStream_t s);

// V [BH, S, D] BF16 (element (b, s, d) at v[b * hs + s * ld + d], D % 32 == 0) -> MXFP8 of V
// transposed, in key blocks of 64: codes [BH, Sp / 64, D, 64] E4M3 and scales [BH, Sp / 64, D, 2],
// Sp = S rounded up to 64, keys past S zero.
hipError_t launch_quant_vt(const uint16_t* v, int64_t BH, int64_t S, int64_t D, int64_t ld, int64_t hs,
                           uint8_t* codes, uint8_t* scales, hipStream_t s);
// Microscaled attention, head dimension 128: Q MXFP4 row-major codes and scales of rows (b, s)
// at b * hs_q + s * ld_q elements (s < Sq), K likewise with ld_k, hs_k (s < Skv); V^T as
// launch_quant_vt writes it for Skv keys; out [BH, Sq, 128] BF16 or FP32 at b * hs_o + s * ld_o.
hipError_t launch_attn_mx(const uint8_t* qc, const uint8_t* qs, int64_t ld_q, int64_t hs_q, const uint8_t* kc,
                          const uint8_t* ks, int64_t ld_k, int64_t hs_k, const uint8_t* vc, const uint8_t* vs,
                          int64_t BH, int64_t Sq, int64_t Skv, float softmax_scale, bool out_f32, void* out,
                          int64_t ld_o, int64_t hs_o, hipStream_t s);

}  // namespace mxk
