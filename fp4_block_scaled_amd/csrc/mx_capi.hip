// C ABI of the library (declared in include/mxfp.h): argument validation, workspace layout and
// dispatch to the gfx950 kernels.  Nothing is launched unless every check passes.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "mx_internal.h"
#include "mxfp.h"

namespace {

thread_local char g_err[512];

mx_status fail(mx_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

mx_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MX_OK;
  return fail(MX_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int group_of(int32_t fmt) { return fmt == MX_FMT_NVFP4 ? 16 : 32; }
bool fmt_ok(int32_t fmt) { return fmt == MX_FMT_MXFP4 || fmt == MX_FMT_MXFP8 || fmt == MX_FMT_NVFP4; }
int64_t code_bytes(int64_t rows, int64_t cols, int32_t fmt) {
  return fmt == MX_FMT_MXFP8 ? rows * cols : rows * (cols / 2);
}
size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
bool is_mx(int32_t fmt) { return fmt == MX_FMT_MXFP4 || fmt == MX_FMT_MXFP8; }
int64_t padded_rows(int64_t rows) { return (rows + 255) / 256 * 256; }
// tiled sizes (MX formats, cols % 128 == 0)
size_t tiled_code_bytes(int64_t rows, int64_t cols, int32_t fmt) { return (size_t)code_bytes(padded_rows(rows), cols, fmt); }
size_t tiled_scale_bytes(int64_t rows, int64_t cols) { return (size_t)(padded_rows(rows) * (cols / 32)); }
// The activation of mx_linear is staged in the tiled layout when the GEMM can use it.
bool act_tiled(int32_t act_fmt, int64_t K) { return is_mx(act_fmt) && K % 128 == 0; }
mx_status check_layout(const mx_qmatrix* q, const char* name) {
  if (q->layout == MX_LAYOUT_ROW_MAJOR) return MX_OK;
  if (q->layout != MX_LAYOUT_TILED) return fail(MX_ERR_UNSUPPORTED, "%s: unknown layout %d", name, q->layout);
  if (!is_mx(q->fmt)) return fail(MX_ERR_UNSUPPORTED, "%s: the tiled layout holds MX formats only", name);
  if (q->cols % 128) return fail(MX_ERR_SHAPE, "%s: the tiled layout needs cols %% 128 == 0", name);
  return MX_OK;
}

struct Workspace {
  uint8_t* codes;
  uint8_t* scales;
  uint16_t* u;
};

size_t ws_code_bytes(int64_t M, int64_t K, int32_t act_fmt) {
  return act_tiled(act_fmt, K) ? tiled_code_bytes(M, K, act_fmt) : (size_t)code_bytes(M, K, act_fmt);
}
size_t ws_scale_bytes(int64_t M, int64_t K, int32_t act_fmt) {
  return act_tiled(act_fmt, K) ? tiled_scale_bytes(M, K) : (size_t)(M * (K / group_of(act_fmt)));
}

Workspace carve(void* ws, int64_t M, int64_t K, int32_t act_fmt, int32_t rank) {
  Workspace w;
  uint8_t* p = (uint8_t*)ws;
  w.codes = p;
  p += round_up(ws_code_bytes(M, K, act_fmt), 256);
  w.scales = p;
  p += round_up(ws_scale_bytes(M, K, act_fmt), 256);
  w.u = rank > 0 ? (uint16_t*)p : nullptr;
  return w;
}

bool finite_pos(float v) { return isfinite(v) && v > 0.0f; }

// Validation shared by mx_linear and mx_linear_q (everything after the activation).
mx_status check_gemm_tail(int32_t act_fmt, int64_t M, int64_t K, const mx_qmatrix* w,
                          const uint16_t* bias, int32_t epilogue, int32_t out_dtype, void* out,
                          int64_t ld_out, uint8_t* out_scales) {
  if (!w) return fail(MX_ERR_NULL, "w is NULL");
  if (!w->codes || !w->scales) return fail(MX_ERR_NULL, "w->codes / w->scales is NULL");
  if (!out && M != 0) return fail(MX_ERR_NULL, "out is NULL");
  if (!fmt_ok(act_fmt) || !fmt_ok(w->fmt)) return fail(MX_ERR_UNSUPPORTED, "unknown format");
  const bool w4_pair = w->fmt == MX_FMT_MXFP4 && (act_fmt == MX_FMT_MXFP4 || act_fmt == MX_FMT_MXFP8);
  const bool w8_pair = w->fmt == MX_FMT_MXFP8 && act_fmt == MX_FMT_MXFP8;
  const bool nv_pair = w->fmt == MX_FMT_NVFP4 && act_fmt == MX_FMT_NVFP4;
  if (!w4_pair && !w8_pair && !nv_pair)
    return fail(MX_ERR_UNSUPPORTED, "format pair (act %d, weight %d) not provided", act_fmt, w->fmt);
  if (M < 0 || K <= 0) return fail(MX_ERR_SHAPE, "M must be >= 0 and K > 0");
  if (w->cols != K) return fail(MX_ERR_SHAPE, "w->cols (%lld) != K (%lld)", (long long)w->cols, (long long)K);
  if (w->rows < 1) return fail(MX_ERR_SHAPE, "w->rows must be >= 1");
  {
    mx_status ls = check_layout(w, "w");
    if (ls != MX_OK) return ls;
  }
  if (K % 32) return fail(MX_ERR_SHAPE, "K (%lld) must be a multiple of 32", (long long)K);
  if (w8_pair && K % 128)
    return fail(MX_ERR_SHAPE, "MXFP8 weights need K %% 128 == 0 (K = %lld)", (long long)K);
  if (M > INT32_MAX || w->rows > INT32_MAX || K > INT32_MAX)
    return fail(MX_ERR_SHAPE, "M, N and K must fit in 31 bits");
  if (nv_pair && !finite_pos(w->global_scale))
    return fail(MX_ERR_SHAPE, "NVFP4 weight global scale must be finite and > 0");
  if (!aligned(w->codes, 16) || !aligned(w->scales, 8))
    return fail(MX_ERR_ALIGN, "weight codes need 16-byte and scales 8-byte alignment");
  if (bias && !aligned(bias, 8)) return fail(MX_ERR_ALIGN, "bias needs 8-byte alignment");
  const int64_t N = w->rows;
  if (epilogue == MX_EPI_BIAS || epilogue == MX_EPI_BIAS_GELU) {
    if (out_dtype != MX_OUT_BF16 && out_dtype != MX_OUT_F32)
      return fail(MX_ERR_UNSUPPORTED, "unknown output dtype %d", out_dtype);
    if (ld_out < N) return fail(MX_ERR_SHAPE, "ld_out (%lld) < N (%lld)", (long long)ld_out, (long long)N);
    if (ld_out % 4) return fail(MX_ERR_ALIGN, "ld_out must be a multiple of 4");
    if (M != 0 && !aligned(out, out_dtype == MX_OUT_F32 ? 16 : 8))
      return fail(MX_ERR_ALIGN, "out is not aligned for vector stores");
  } else if (epilogue == MX_EPI_BIAS_GELU_QUANT_MXFP4) {
    if (!out_scales && M != 0) return fail(MX_ERR_NULL, "out_scales is NULL");
    if (N % 32) return fail(MX_ERR_SHAPE, "re-quantizing epilogue needs N %% 32 == 0");
    if (ld_out != N) return fail(MX_ERR_SHAPE, "re-quantizing epilogue needs ld_out == N");
    if (M != 0 && !aligned(out, 8)) return fail(MX_ERR_ALIGN, "out codes need 8-byte alignment");
  } else if (epilogue == MX_EPI_BIAS_GELU_QUANT_MXFP4_TILED) {
    if (act_fmt != MX_FMT_MXFP4) return fail(MX_ERR_UNSUPPORTED, "tiled re-quantized output needs MXFP4 activations");
    if (!out_scales && M != 0) return fail(MX_ERR_NULL, "out_scales is NULL");
    if (N % 128 || K % 128) return fail(MX_ERR_SHAPE, "tiled re-quantized output needs N %% 128 == 0 and K %% 128 == 0");
    if (ld_out != N) return fail(MX_ERR_SHAPE, "re-quantizing epilogue needs ld_out == N");
    if (M != 0 && (!aligned(out, 16) || !aligned(out_scales, 16)))
      return fail(MX_ERR_ALIGN, "tiled output codes and scales need 16-byte alignment");
  } else {
    return fail(MX_ERR_UNSUPPORTED, "unknown epilogue %d", epilogue);
  }
  return MX_OK;
}

}  // namespace

extern "C" {

int mx_abi_version(void) { return MX_ABI_VERSION; }

const char* mx_status_string(int status) {
  switch (status) {
    case MX_OK: return "MX_OK";
    case MX_ERR_NULL: return "MX_ERR_NULL";
    case MX_ERR_SHAPE: return "MX_ERR_SHAPE";
    case MX_ERR_ALIGN: return "MX_ERR_ALIGN";
    case MX_ERR_UNSUPPORTED: return "MX_ERR_UNSUPPORTED";
    case MX_ERR_WORKSPACE: return "MX_ERR_WORKSPACE";
    case MX_ERR_HIP: return "MX_ERR_HIP";
    default: return "MX_UNKNOWN_STATUS";
  }
}

const char* mx_last_error(void) { return g_err; }

float mx_nvfp4_global_scale(float amax) {
  if (!(amax > 0.0f) || !isfinite(amax)) return 1.0f;
  volatile float num = amax, den = 2688.0f;  // 6 (max E2M1) * 448 (max E4M3)
  return num / den;
}

mx_status mx_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int32_t fmt,
                      int32_t layout, float global_scale, void* codes, uint8_t* scales,
                      void* stream) {
  g_err[0] = 0;
  if (!fmt_ok(fmt)) return fail(MX_ERR_UNSUPPORTED, "unknown format %d", fmt);
  if (layout != MX_LAYOUT_ROW_MAJOR && layout != MX_LAYOUT_TILED)
    return fail(MX_ERR_UNSUPPORTED, "unknown layout %d", layout);
  const bool tiled = layout == MX_LAYOUT_TILED;
  if (tiled && !is_mx(fmt)) return fail(MX_ERR_UNSUPPORTED, "the tiled layout holds MX formats only");
  if (tiled && cols % 128) return fail(MX_ERR_SHAPE, "the tiled layout needs cols %% 128 == 0");
  const int G = group_of(fmt);
  if (rows < 0 || cols <= 0) return fail(MX_ERR_SHAPE, "rows must be >= 0 and cols > 0");
  if (cols % G) return fail(MX_ERR_SHAPE, "cols (%lld) must be a multiple of %d", (long long)cols, G);
  if (ld_x < cols) return fail(MX_ERR_SHAPE, "ld_x < cols");
  if (fmt == MX_FMT_NVFP4 && !finite_pos(global_scale))
    return fail(MX_ERR_SHAPE, "NVFP4 global scale must be finite and > 0");
  if (rows == 0) return MX_OK;
  if (!x || !codes || !scales) return fail(MX_ERR_NULL, "x, codes and scales must be non-NULL");
  if (!aligned(x, 16) || ld_x % 8) return fail(MX_ERR_ALIGN, "x needs 16-byte alignment and ld_x %% 8 == 0");
  if (!aligned(codes, fmt == MX_FMT_MXFP8 ? 8 : 4)) return fail(MX_ERR_ALIGN, "codes misaligned");
  hipStream_t s = (hipStream_t)stream;
  if (tiled) {
    if (!aligned(codes, 16) || !aligned(scales, 16)) return fail(MX_ERR_ALIGN, "tiled codes and scales need 16-byte alignment");
    return hip_status(mxk::launch_quant_mx_tiled(x, rows, cols, ld_x, fmt == MX_FMT_MXFP8 ? 1 : 0,
                                                 (uint8_t*)codes, scales, s), "mx_quantize launch");
  }
  hipError_t e = fmt == MX_FMT_NVFP4
                     ? mxk::launch_quant_nv(x, rows, cols, ld_x, global_scale, (uint8_t*)codes, scales, s)
                     : mxk::launch_quant_mx(x, rows, cols, ld_x, fmt == MX_FMT_MXFP8 ? 1 : 0,
                                            (uint8_t*)codes, scales, s);
  return hip_status(e, "mx_quantize launch");
}

// Checks shared by mx_norm and mx_norm_quantize (the input side).
static mx_status check_norm_in(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, float eps,
                               const float* gamma, const float* beta, const float* scale,
                               const float* shift) {
  if (rows < 0 || cols <= 0 || cols % 32) return fail(MX_ERR_SHAPE, "rows >= 0 and cols %% 32 == 0 (cols > 0) needed");
  if (cols > MX_NORM_MAX_COLS) return fail(MX_ERR_SHAPE, "cols (%lld) > %d", (long long)cols, MX_NORM_MAX_COLS);
  if (ld_x < cols) return fail(MX_ERR_SHAPE, "ld_x < cols");
  if (!(eps > 0.0f) || !isfinite(eps)) return fail(MX_ERR_SHAPE, "eps must be finite and > 0");
  const float* vecs[4] = {gamma, beta, scale, shift};
  for (const float* v : vecs)
    if (v && !aligned(v, 4)) return fail(MX_ERR_ALIGN, "gamma / beta / scale / shift need 4-byte alignment");
  if (rows != 0 && !x) return fail(MX_ERR_NULL, "x is NULL");
  if (rows != 0 && (!aligned(x, 16) || ld_x % 8)) return fail(MX_ERR_ALIGN, "x needs 16-byte alignment and ld_x %% 8 == 0");
  return MX_OK;
}

mx_status mx_norm(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, float eps,
                  const float* gamma, const float* beta, const float* scale, const float* shift,
                  uint16_t* y, int64_t ld_y, void* stream) {
  g_err[0] = 0;
  mx_status st = check_norm_in(x, rows, cols, ld_x, eps, gamma, beta, scale, shift);
  if (st != MX_OK) return st;
  if (ld_y < cols) return fail(MX_ERR_SHAPE, "ld_y < cols");
  if (rows == 0) return MX_OK;
  if (!y) return fail(MX_ERR_NULL, "y is NULL");
  if (!aligned(y, 16) || ld_y % 8) return fail(MX_ERR_ALIGN, "y needs 16-byte alignment and ld_y %% 8 == 0");
  return hip_status(mxk::launch_norm_quant(x, rows, cols, ld_x, eps, gamma, beta, scale, shift, 0, 0, y,
                                           ld_y, nullptr, nullptr, (hipStream_t)stream),
                    "mx_norm launch");
}

mx_status mx_norm_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, float eps,
                           const float* gamma, const float* beta, const float* scale,
                           const float* shift, int32_t fmt, int32_t layout, void* codes,
                           uint8_t* scales, void* stream) {
  g_err[0] = 0;
  if (fmt != MX_FMT_MXFP4 && fmt != MX_FMT_MXFP8)
    return fail(MX_ERR_UNSUPPORTED, "mx_norm_quantize writes MXFP4 or MXFP8 (format %d)", fmt);
  if (layout != MX_LAYOUT_ROW_MAJOR && layout != MX_LAYOUT_TILED)
    return fail(MX_ERR_UNSUPPORTED, "unknown layout %d", layout);
  const bool tiled = layout == MX_LAYOUT_TILED;
  mx_status st = check_norm_in(x, rows, cols, ld_x, eps, gamma, beta, scale, shift);
  if (st != MX_OK) return st;
  if (tiled && cols % 128) return fail(MX_ERR_SHAPE, "the tiled layout needs cols %% 128 == 0");
  if (rows == 0) return MX_OK;
  if (!codes || !scales) return fail(MX_ERR_NULL, "codes and scales must be non-NULL");
  if (tiled ? !aligned(codes, 16) || !aligned(scales, 16) : !aligned(codes, fmt == MX_FMT_MXFP8 ? 8 : 4))
    return fail(MX_ERR_ALIGN, tiled ? "tiled codes and scales need 16-byte alignment" : "codes misaligned");
  return hip_status(mxk::launch_norm_quant(x, rows, cols, ld_x, eps, gamma, beta, scale, shift,
                                           tiled ? 2 : 1, fmt == MX_FMT_MXFP8 ? 1 : 0, nullptr, 0,
                                           (uint8_t*)codes, scales, (hipStream_t)stream),
                    "mx_norm_quantize launch");
}

mx_status mx_quantize_vt(const uint16_t* v, int64_t BH, int64_t S, int64_t D, int64_t ld_v,
                         int64_t hs_v, uint8_t* codes, uint8_t* scales, void* stream) {
  g_err[0] = 0;
  if (BH < 0 || BH > 65535 || S < 0 || S > (1 << 24)) return fail(MX_ERR_SHAPE, "need 0 <= BH <= 65535 and 0 <= S <= 2^24");
  if (D <= 0 || D % 32) return fail(MX_ERR_SHAPE, "D (%lld) must be a positive multiple of 32", (long long)D);
  if (ld_v < D || ld_v % 8 || hs_v < 0 || hs_v % 8) return fail(MX_ERR_ALIGN, "need ld_v >= D and ld_v, hs_v multiples of 8");
  if (BH == 0 || S == 0) return MX_OK;
  if (!v || !codes || !scales) return fail(MX_ERR_NULL, "v, codes and scales must be non-NULL");
  if (!aligned(v, 16) || !aligned(codes, 16)) return fail(MX_ERR_ALIGN, "v and codes need 16-byte alignment");
  return hip_status(mxk::launch_quant_vt(v, BH, S, D, ld_v, hs_v, codes, scales, (hipStream_t)stream),
                    "mx_quantize_vt launch");
}

mx_status mx_attention(const uint8_t* q_codes, const uint8_t* q_scales, int64_t ld_q, int64_t hs_q,
                       const uint8_t* k_codes, const uint8_t* k_scales, int64_t ld_k, int64_t hs_k,
                       const uint8_t* vt_codes, const uint8_t* vt_scales, int64_t BH, int64_t S_q,
                       int64_t S_kv, int64_t D, float softmax_scale, int32_t out_dtype, void* out,
                       int64_t ld_o, int64_t hs_o, void* stream) {
  g_err[0] = 0;
  if (D != MX_ATTN_HEAD_DIM) return fail(MX_ERR_UNSUPPORTED, "head dimension %lld (only %d)", (long long)D, MX_ATTN_HEAD_DIM);
  if (BH < 0 || BH > 65535 || S_q < 0 || S_q > (1 << 24) || S_kv < 0 || S_kv > (1 << 24))
    return fail(MX_ERR_SHAPE, "need 0 <= BH <= 65535 and 0 <= S_q, S_kv <= 2^24");
  if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return fail(MX_ERR_SHAPE, "softmax_scale must be finite and > 0");
  if (out_dtype != MX_OUT_BF16 && out_dtype != MX_OUT_F32) return fail(MX_ERR_UNSUPPORTED, "unknown out_dtype %d", out_dtype);
  if (ld_q < D || ld_q % 128 || hs_q < 0 || hs_q % 128 || ld_k < D || ld_k % 128 || hs_k < 0 || hs_k % 128)
    return fail(MX_ERR_ALIGN, "need ld_q, ld_k >= 128 and ld_q, hs_q, ld_k, hs_k multiples of 128");
  if (ld_o < D || ld_o % 8 || hs_o < 0 || hs_o % 8) return fail(MX_ERR_ALIGN, "need ld_o >= 128 and ld_o, hs_o multiples of 8");
  if ((S_kv + 64) * (ld_k / 2) >= (int64_t)1 << 32) return fail(MX_ERR_SHAPE, "(S_kv + 64) * ld_k / 2 must stay below 2^32");
  if (BH == 0 || S_q == 0) return MX_OK;
  if (S_kv == 0) return fail(MX_ERR_SHAPE, "attention over zero keys is undefined (S_kv == 0, S_q > 0)");
  if (!q_codes || !q_scales || !k_codes || !k_scales || !vt_codes || !vt_scales || !out)
    return fail(MX_ERR_NULL, "operands and out must be non-NULL");
  if (!aligned(q_codes, 16) || !aligned(k_codes, 16) || !aligned(vt_codes, 16) || !aligned(out, 16) ||
      !aligned(q_scales, 4) || !aligned(k_scales, 4) || !aligned(vt_scales, 4))
    return fail(MX_ERR_ALIGN, "codes and out need 16-byte, scales 4-byte alignment");
  return hip_status(mxk::launch_attn_mx(q_codes, q_scales, ld_q, hs_q, k_codes, k_scales, ld_k, hs_k, vt_codes,
                                        vt_scales, BH, S_q, S_kv, softmax_scale, out_dtype == MX_OUT_F32, out,
                                        ld_o, hs_o, (hipStream_t)stream),
                    "mx_attention launch");
}

mx_status mx_tiled_bytes(int64_t rows, int64_t cols, int32_t fmt, size_t* code_bytes_out,
                         size_t* scale_bytes_out) {
  g_err[0] = 0;
  if (!code_bytes_out || !scale_bytes_out) return fail(MX_ERR_NULL, "output pointers must be non-NULL");
  if (!is_mx(fmt)) return fail(MX_ERR_UNSUPPORTED, "the tiled layout holds MX formats only");
  if (rows < 0 || cols <= 0 || cols % 128) return fail(MX_ERR_SHAPE, "rows >= 0 and cols %% 128 == 0 needed");
  *code_bytes_out = tiled_code_bytes(rows, cols, fmt);
  *scale_bytes_out = tiled_scale_bytes(rows, cols);
  return MX_OK;
}

mx_status mx_relayout(const mx_qmatrix* src, const mx_qmatrix* dst, void* stream) {
  g_err[0] = 0;
  if (!src || !dst) return fail(MX_ERR_NULL, "src and dst must be non-NULL");
  if (src->fmt != dst->fmt || src->rows != dst->rows || src->cols != dst->cols)
    return fail(MX_ERR_SHAPE, "src and dst differ in format or shape");
  if (!is_mx(src->fmt)) return fail(MX_ERR_UNSUPPORTED, "the tiled layout holds MX formats only");
  mx_status ls = check_layout(src, "src");
  if (ls == MX_OK) ls = check_layout(dst, "dst");
  if (ls != MX_OK) return ls;
  if (src->layout == dst->layout) return fail(MX_ERR_UNSUPPORTED, "src and dst have the same layout");
  if (src->rows < 0 || src->cols <= 0) return fail(MX_ERR_SHAPE, "bad rows/cols");
  if (src->rows == 0) return MX_OK;
  if (!src->codes || !src->scales || !dst->codes || !dst->scales)
    return fail(MX_ERR_NULL, "codes and scales must be non-NULL");
  if (!aligned(src->codes, 16) || !aligned(dst->codes, 16) || !aligned(src->scales, 4) || !aligned(dst->scales, 4))
    return fail(MX_ERR_ALIGN, "codes need 16-byte and scales 4-byte alignment");
  return hip_status(mxk::launch_relayout((const uint8_t*)src->codes, src->scales, (uint8_t*)dst->codes,
                                         (uint8_t*)dst->scales, src->rows, src->cols,
                                         src->fmt == MX_FMT_MXFP8 ? 1 : 0,
                                         dst->layout == MX_LAYOUT_TILED, (hipStream_t)stream),
                    "mx_relayout launch");
}

mx_status mx_dequantize(const mx_qmatrix* q, uint16_t* y, int64_t ld_y, void* stream) {
  g_err[0] = 0;
  if (!q) return fail(MX_ERR_NULL, "q is NULL");
  if (!fmt_ok(q->fmt)) return fail(MX_ERR_UNSUPPORTED, "unknown format %d", q->fmt);
  if (q->layout != MX_LAYOUT_ROW_MAJOR)
    return fail(MX_ERR_UNSUPPORTED, "mx_dequantize reads row-major matrices (see mx_relayout)");
  const int G = group_of(q->fmt);
  if (q->rows < 0 || q->cols <= 0 || q->cols % G) return fail(MX_ERR_SHAPE, "bad rows/cols");
  if (ld_y < q->cols) return fail(MX_ERR_SHAPE, "ld_y < cols");
  if (q->fmt == MX_FMT_NVFP4 && !finite_pos(q->global_scale))
    return fail(MX_ERR_SHAPE, "NVFP4 global scale must be finite and > 0");
  if (q->rows == 0) return MX_OK;
  if (!q->codes || !q->scales || !y) return fail(MX_ERR_NULL, "codes, scales and y must be non-NULL");
  if (!aligned(y, 16) || ld_y % 8) return fail(MX_ERR_ALIGN, "y needs 16-byte alignment and ld_y %% 8 == 0");
  if (!aligned(q->codes, q->fmt == MX_FMT_MXFP8 ? 8 : 4)) return fail(MX_ERR_ALIGN, "codes misaligned");
  hipError_t e = mxk::launch_dequant((const uint8_t*)q->codes, q->scales, q->rows, q->cols, q->fmt,
                                     q->global_scale, y, ld_y, (hipStream_t)stream);
  return hip_status(e, "mx_dequantize launch");
}

mx_status mx_absmax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, float* amax,
                    void* stream) {
  g_err[0] = 0;
  if (!x || !amax) return fail(MX_ERR_NULL, "x and amax must be non-NULL");
  if (rows < 0 || cols < 0 || ld_x < cols) return fail(MX_ERR_SHAPE, "bad rows/cols/ld_x");
  if (!aligned(amax, 4)) return fail(MX_ERR_ALIGN, "amax misaligned");
  return hip_status(mxk::launch_absmax(x, rows, cols, ld_x, amax, (hipStream_t)stream),
                    "mx_absmax launch");
}

size_t mx_linear_workspace_bytes(int64_t M, int64_t K, int32_t act_fmt, int32_t rank) {
  if (M <= 0 || K <= 0 || !fmt_ok(act_fmt)) return 0;
  size_t b = round_up(ws_code_bytes(M, K, act_fmt), 256) + round_up(ws_scale_bytes(M, K, act_fmt), 256);
  if (rank > 0) b += round_up((size_t)M * (size_t)rank * 2, 256);
  return b;
}

static mxk::GemmParams gemm_params(const uint8_t* a_codes, const uint8_t* a_scales, float a_gscale,
                                   bool a_is_tiled, int64_t M, int64_t K, const mx_qmatrix* w,
                                   const uint16_t* bias, const uint16_t* lr_u, const mx_lowrank* lr,
                                   int32_t epilogue, int32_t out_dtype, void* out, int64_t ld_out,
                                   uint8_t* out_scales) {
  mxk::GemmParams p;
  p.a_codes = a_codes;
  p.a_scales = a_scales;
  p.w_codes = (const uint8_t*)w->codes;
  p.w_scales = w->scales;
  p.bias = bias;
  p.lr_u = lr_u;
  p.lr_up = lr ? lr->up : nullptr;
  p.R = lr ? lr->rank : 0;
  p.out = out;
  p.out_scales = out_scales;
  p.ld_out = ld_out;
  p.out_scale = w->fmt == MX_FMT_NVFP4 ? a_gscale * w->global_scale : 1.0f;
  p.M = (int)M;
  p.N = (int)w->rows;
  p.K = (int)K;
  p.epi = epilogue == MX_EPI_BIAS ? mxk::EPI_BIAS
          : epilogue == MX_EPI_BIAS_GELU ? mxk::EPI_GELU
          : epilogue == MX_EPI_BIAS_GELU_QUANT_MXFP4 ? mxk::EPI_GELU_QUANT : mxk::EPI_GELU_QUANT_T;
  p.out_f32 = out_dtype == MX_OUT_F32 ? 1 : 0;
  p.a_tiled = a_is_tiled ? 1 : 0;
  p.w_tiled = w->layout == MX_LAYOUT_TILED ? 1 : 0;
  return p;
}

static mx_status run_gemm(const uint8_t* a_codes, const uint8_t* a_scales, float a_gscale,
                          int32_t act_fmt, bool a_is_tiled, int64_t M, int64_t K, const mx_qmatrix* w,
                          const uint16_t* bias, const uint16_t* lr_u, const mx_lowrank* lr,
                          int32_t epilogue, int32_t out_dtype, void* out, int64_t ld_out,
                          uint8_t* out_scales, hipStream_t s) {
  const mxk::GemmParams p = gemm_params(a_codes, a_scales, a_gscale, a_is_tiled, M, K, w, bias, lr_u, lr,
                                        epilogue, out_dtype, out, ld_out, out_scales);
  hipError_t e = w->fmt == MX_FMT_NVFP4 ? mxk::launch_gemm_nv(p, s)
                                         : mxk::launch_gemm_mx(p, act_fmt == MX_FMT_MXFP8, w->fmt == MX_FMT_MXFP8, s);
  return hip_status(e, "GEMM launch");
}

}  // extern "C"

namespace {

// Arguments of mx_linear besides the workspace (shared with mx_linear_noalloc).
mx_status check_linear(const uint16_t* a, int64_t M, int64_t K, int64_t ld_a, int32_t act_fmt,
                       float act_global_scale, const mx_qmatrix* w, const uint16_t* bias,
                       const mx_lowrank* lr, int32_t epilogue, int32_t out_dtype, void* out,
                       int64_t ld_out, uint8_t* out_scales) {
  mx_status st = check_gemm_tail(act_fmt, M, K, w, bias, epilogue, out_dtype, out, ld_out, out_scales);
  if (st != MX_OK) return st;
  if (!a && M != 0) return fail(MX_ERR_NULL, "a is NULL");
  if (ld_a < K) return fail(MX_ERR_SHAPE, "ld_a < K");
  if ((M != 0 && !aligned(a, 16)) || ld_a % 8)
    return fail(MX_ERR_ALIGN, "a needs 16-byte alignment and ld_a %% 8 == 0");
  if (act_fmt == MX_FMT_NVFP4 && !finite_pos(act_global_scale))
    return fail(MX_ERR_SHAPE, "NVFP4 activation global scale must be finite and > 0");
  if (lr) {
    if (act_fmt == MX_FMT_NVFP4) return fail(MX_ERR_UNSUPPORTED, "low-rank branch needs an MX format");
    if (!lr->down || !lr->up) return fail(MX_ERR_NULL, "lr->down / lr->up is NULL");
    if (lr->rank < 1 || lr->rank > 64 || lr->rank % 16) return fail(MX_ERR_SHAPE, "rank must be 16, 32, 48 or 64");
    if (!aligned(lr->down, 16) || !aligned(lr->up, 16)) return fail(MX_ERR_ALIGN, "low-rank factors need 16-byte alignment");
    if (31 * ld_a + K >= ((int64_t)1 << 30))
      return fail(MX_ERR_SHAPE, "with a low-rank branch, 31 * ld_a + K must be below 2^30");
  }
  return MX_OK;
}

// The launches of mx_linear on a checked argument set and a workspace of
// mx_linear_workspace_bytes bytes (256-byte aligned).
mx_status run_linear(const uint16_t* a, int64_t M, int64_t K, int64_t ld_a, int32_t act_fmt,
                     float act_global_scale, const mx_qmatrix* w, const uint16_t* bias,
                     const mx_lowrank* lr, int32_t epilogue, int32_t out_dtype, void* out,
                     int64_t ld_out, uint8_t* out_scales, void* workspace, hipStream_t s) {
  const int32_t rank = lr ? lr->rank : 0;
  if (act_fmt == MX_FMT_MXFP4 && w->fmt == MX_FMT_MXFP4 && rank == 0 && M > 0) {
    // a small grid: quantization and GEMM in one launch (same output bits)
    const mxk::GemmParams p = gemm_params(nullptr, nullptr, 1.0f, false, M, K, w, bias, nullptr, nullptr,
                                          epilogue, out_dtype, out, ld_out, out_scales);
    if (mxk::linear_fused_small_ok(p))
      return hip_status(mxk::launch_linear_fused_small(p, a, ld_a, s), "small linear launch");
  }
  Workspace ws = carve(workspace, M, K, act_fmt, rank);
  hipError_t e;
  const bool tiled = act_tiled(act_fmt, K);
  if (rank > 0 && tiled && act_fmt == MX_FMT_MXFP8) {
    // W4A8 SVDQuant: one pass over a quantizes it and computes the low-rank input u.  Tiled
    // padding rows past the last 32-row block stay unwritten in the workspace: they only feed
    // output rows >= M, which are never stored.
    e = mxk::launch_quant8_lowrank_down(a, ld_a, lr->down, (int)M, (int)K, rank, ws.u, ws.codes, ws.scales, s);
    if (e != hipSuccess) return hip_status(e, "quantizer + low-rank launch");
  } else {
    if (act_fmt == MX_FMT_NVFP4)
      e = mxk::launch_quant_nv(a, M, K, ld_a, act_global_scale, ws.codes, ws.scales, s);
    else if (tiled)
      e = mxk::launch_quant_mx_tiled(a, M, K, ld_a, act_fmt == MX_FMT_MXFP8 ? 1 : 0, ws.codes, ws.scales, s);
    else
      e = mxk::launch_quant_mx(a, M, K, ld_a, act_fmt == MX_FMT_MXFP8 ? 1 : 0, ws.codes, ws.scales, s);
    if (e != hipSuccess) return hip_status(e, "activation quantizer launch");
    if (rank > 0) {
      e = mxk::launch_lowrank_down(a, ld_a, lr->down, (int)M, (int)K, rank, ws.u, s);
      if (e != hipSuccess) return hip_status(e, "low-rank launch");
    }
  }
  return run_gemm(ws.codes, ws.scales, act_global_scale, act_fmt, tiled, M, K, w, bias, ws.u, lr,
                  epilogue, out_dtype, out, ld_out, out_scales, s);
}

// ---------------------------------------------------------------------------------------------
// The statically allocated workspace of mx_linear_noalloc: one copy per GPU, held until the
// process ends.  In host code `scratch` names a host-side stand-in, not device memory: its
// device address is taken once per device with hipGetSymbolAddress (with that device current)
// and only that address is used.
// ---------------------------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[MX_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once taken

mx_status scratch_address(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MX_ERR_HIP, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p || !aligned(p, 256)) return fail(MX_ERR_HIP, "scratch symbol has no usable device address");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MX_OK;
}

}  // namespace

extern "C" {

mx_status mx_linear(const uint16_t* a, int64_t M, int64_t K, int64_t ld_a, int32_t act_fmt,
                    float act_global_scale, const mx_qmatrix* w, const uint16_t* bias,
                    const mx_lowrank* lr, int32_t epilogue, int32_t out_dtype, void* out,
                    int64_t ld_out, uint8_t* out_scales, void* workspace, size_t workspace_bytes,
                    void* stream) {
  g_err[0] = 0;
  mx_status st = check_linear(a, M, K, ld_a, act_fmt, act_global_scale, w, bias, lr, epilogue, out_dtype,
                              out, ld_out, out_scales);
  if (st != MX_OK) return st;
  if (M == 0) return MX_OK;
  const size_t need = mx_linear_workspace_bytes(M, K, act_fmt, lr ? lr->rank : 0);
  if (!workspace || workspace_bytes < need)
    return fail(MX_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (!aligned(workspace, 256)) return fail(MX_ERR_ALIGN, "workspace needs 256-byte alignment");
  return run_linear(a, M, K, ld_a, act_fmt, act_global_scale, w, bias, lr, epilogue, out_dtype, out,
                    ld_out, out_scales, workspace, (hipStream_t)stream);
}

mx_status mx_linear_noalloc(const uint16_t* a, int64_t M, int64_t K, int64_t ld_a, int32_t act_fmt,
                            float act_global_scale, const mx_qmatrix* w, const uint16_t* bias,
                            const mx_lowrank* lr, int32_t epilogue, int32_t out_dtype, void* out,
                            int64_t ld_out, uint8_t* out_scales, void* stream) {
  g_err[0] = 0;
  mx_status st = check_linear(a, M, K, ld_a, act_fmt, act_global_scale, w, bias, lr, epilogue, out_dtype,
                              out, ld_out, out_scales);
  if (st != MX_OK) return st;
  if (M == 0) return MX_OK;
  const size_t need = mx_linear_workspace_bytes(M, K, act_fmt, lr ? lr->rank : 0);
  if (need > (size_t)MX_NOALLOC_SCRATCH_BYTES)
    return fail(MX_ERR_WORKSPACE, "workspace of %zu bytes needed, the static scratch holds %zu", need,
                (size_t)MX_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != MX_OK) return st;
  return run_linear(a, M, K, ld_a, act_fmt, act_global_scale, w, bias, lr, epilogue, out_dtype, out,
                    ld_out, out_scales, ws, (hipStream_t)stream);
}

mx_status mx_linear_q(const mx_qmatrix* a, const mx_qmatrix* w, const uint16_t* bias,
                      int32_t epilogue, int32_t out_dtype, void* out, int64_t ld_out,
                      uint8_t* out_scales, void* stream) {
  g_err[0] = 0;
  if (!a) return fail(MX_ERR_NULL, "a is NULL");
  mx_status st = check_gemm_tail(a->fmt, a->rows, a->cols, w, bias, epilogue, out_dtype, out,
                                 ld_out, out_scales);
  if (st != MX_OK) return st;
  st = check_layout(a, "a");
  if (st != MX_OK) return st;
  if (a->rows == 0) return MX_OK;
  if (!a->codes || !a->scales) return fail(MX_ERR_NULL, "a->codes / a->scales is NULL");
  if (!aligned(a->codes, 16) || !aligned(a->scales, 8))
    return fail(MX_ERR_ALIGN, "activation codes need 16-byte and scales 8-byte alignment");
  if (a->fmt == MX_FMT_NVFP4 && !finite_pos(a->global_scale))
    return fail(MX_ERR_SHAPE, "NVFP4 activation global scale must be finite and > 0");
  return run_gemm((const uint8_t*)a->codes, a->scales, a->global_scale, a->fmt,
                  a->layout == MX_LAYOUT_TILED, a->rows, a->cols,
                  w, bias, nullptr, nullptr, epilogue, out_dtype, out, ld_out, out_scales,
                  (hipStream_t)stream);
}

}  // extern "C"
