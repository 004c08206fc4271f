/*
 * mxfp.h - C ABI of the MI355X (gfx950) microscaled-FP4 linear layer.
 *
 * What it computes (model cards of quantized Wan2.2 transformers):
 *  - "Wan2.2-I2V-A14B-Lightning-Diffusers-MXFP4-AutoRound", Quantization Details, and
 *    "Wan2.2-Animate-14B-Diffusers-MXFP4-AutoRound", Quantization Details: W4A4 MXFP4 linear
 *    layers; weights are FP4 E2M1 codes packed two per byte with one E8M0 scale per 32
 *    consecutive input channels; activations are quantized to MXFP4 dynamically at run time;
 *    biases are F16.
 *  - "Wan2.2-T2V-A14B-Diffusers-NVFP4-AutoRound", Model Details: NVFP4 variant, E2M1 codes with
 *    one FP8 E4M3 scale per 16 and one FP32 global scale per tensor; activation block scales
 *    dynamic, activation global scale static.
 *  - "Wan2.2 W4A8 SVDQuant - NVIDIA (CUDA) artifacts": W4A8 variant, MXFP4 weights times
 *    dynamically quantized MXFP8 (E4M3, per-32 E8M0) activations plus a rank-32 low-rank branch
 *    with BF16 factors.
 *  - "Wan2.2-I2V-A14B-Lightning-Diffusers-MXFP4-AutoRound", VBench-I2V results and Performance
 *    Profile: MXFP8 linear layers (E4M3 weights and activations, per-32 E8M0 scales) are the
 *    quality and speed reference the MXFP4 layers are compared with (W8A8).
 * The bit-level encodings follow OCP Microscaling (MX) v1.0: the shared exponent of a block is
 * floor(log2(max|x|)) - emax(element) (emax 2 for E2M1, 8 for E4M3), elements are rounded to
 * nearest-even with saturation, signs are kept.  NVFP4 stores its global scale in the decode
 * direction: value = code * block_scale * global_scale.
 *
 * Conventions for every call:
 *  - Pointers marked "device" are HIP device (or host-coherent) addresses owned by the caller;
 *    the library allocates nothing, frees nothing and keeps no pointer after the call returns
 *    (mx_linear_noalloc's workspace is a static device array of the library, see there).
 *  - BF16 and FP16 values are passed as uint16_t bit patterns.
 *  - The canonical layout (MX_LAYOUT_ROW_MAJOR) is row-major and unshuffled.  FP4 codes:
 *    [rows, cols/2] bytes, element 2j in the low nibble of byte j.  FP8 codes: [rows, cols]
 *    bytes.  Scales: [rows, cols/G] bytes with G = 32 (E8M0, MX formats) or G = 16 (E4M3,
 *    NVFP4); groups start at column 0.
 *  - MX_LAYOUT_TILED (MXFP4 / MXFP8 only, cols % 128 == 0) is the GEMM operand layout: the
 *    same bytes regrouped so that every 1 KB of codes and every 256 bytes of scales that the
 *    GEMM stages together are contiguous.  Rows are padded to Rp = rows rounded up to 256; the
 *    padding rows hold zero codes and zero scale bytes.  With nkc = cols / 128:
 *      FP4 codes: 1 KB tile (rb, kb) = rows 16rb..16rb+15, columns 128kb..128kb+127, at byte
 *        (rb * nkc + kb) * 1024; row r of the tile at 64r; its 16-byte column group g (32
 *        elements, nibbles packed as above) at 16 * (g ^ ((r >> 2) & 3)).
 *      FP8 codes: 1 KB tile (rb, kb) = rows 8rb..8rb+7, at byte (rb * nkc + kb) * 1024; row r
 *        of the tile at 128r; its 16-byte column group g (16 elements) at 16 * (g ^ (((8rb +
 *        r) >> 1) & 7)).
 *      Scales: 256-byte tile (sb, kb) = rows 64sb..64sb+63 at byte (sb * nkc + kb) * 256; row
 *        r of the tile at 4r: the four scale bytes of columns 128kb..128kb+127 in order.
 *    Sizes: codes Rp * cols / 2 (FP4) or Rp * cols (FP8) bytes, scales Rp * cols / 32 bytes.
 *  - A linear layer computes y[m, n] = sum_k a[m, k] * w[n, k] + bias[n]: the weight is N x K
 *    with K contiguous ("TN"); the output is M x N.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls are asynchronous on that
 *    stream; results are valid once the caller synchronises it.
 *  - Errors: every argument is validated before anything is launched, so on an error nothing is
 *    written.  MX_ERR_HIP reports a launch failure.  mx_last_error() gives a message for the
 *    calling thread's last failing call.  M = 0 (rows = 0) is a valid no-op.
 *  - Results are deterministic: no atomics, no split-K; the same inputs give the same bytes.
 *  - Calls are thread-safe; the library holds no state besides the per-thread error message
 *    and mx_linear_noalloc's per-GPU static workspace (whose concurrent use races, see there).
 */
#ifndef MXFP_H
#define MXFP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MX_ABI_VERSION 2

typedef enum mx_status {
    MX_OK = 0,
    MX_ERR_NULL = 1,        /* a required pointer is NULL */
    MX_ERR_SHAPE = 2,       /* sizes inconsistent or not a multiple of the group size */
    MX_ERR_ALIGN = 3,       /* a pointer or leading dimension breaks the alignment rule */
    MX_ERR_UNSUPPORTED = 4, /* format / epilogue / output combination not provided */
    MX_ERR_WORKSPACE = 5,   /* workspace missing or smaller than mx_linear_workspace_bytes */
    MX_ERR_HIP = 6          /* a HIP launch failed */
} mx_status;

typedef enum mx_format {
    MX_FMT_MXFP4 = 0, /* E2M1 codes, E8M0 scale per 32 */
    MX_FMT_MXFP8 = 1, /* E4M3 codes, E8M0 scale per 32 */
    MX_FMT_NVFP4 = 2  /* E2M1 codes, E4M3 scale per 16, FP32 global scale */
} mx_format;

typedef enum mx_epilogue {
    MX_EPI_BIAS = 0,                 /* y = acc + bias */
    MX_EPI_BIAS_GELU = 1,            /* y = gelu_tanh(acc + bias) */
    MX_EPI_BIAS_GELU_QUANT_MXFP4 = 2, /* h = gelu_tanh(acc + bias), re-quantized to MXFP4 along N */
    MX_EPI_BIAS_GELU_QUANT_MXFP4_TILED = 3 /* the same, written in the tiled layout */
} mx_epilogue;

typedef enum mx_out_dtype { MX_OUT_BF16 = 0, MX_OUT_F32 = 1 } mx_out_dtype;

typedef enum mx_layout {
    MX_LAYOUT_ROW_MAJOR = 0, /* canonical */
    MX_LAYOUT_TILED = 1      /* GEMM operand layout (see above) */
} mx_layout;

/* A quantized matrix (rows x cols logical elements) in one of the layouts above. */
typedef struct mx_qmatrix {
    const void* codes;     /* device */
    const uint8_t* scales; /* device */
    float global_scale;    /* NVFP4 only: decode-direction FP32 global scale; ignored for MX */
    int32_t fmt;           /* mx_format */
    int64_t rows;
    int64_t cols;
    int32_t layout;        /* mx_layout */
} mx_qmatrix;

/* Low-rank branch of SVDQuant ("Wan2.2 W4A8 SVDQuant", Contents/Accuracy: rank-32 BF16
 * factors).  y += bf16(x . L_down) . L_up, x being the unquantized BF16 activation, L_down the
 * K x rank and L_up the rank x N factor; both are passed transposed so that the summed index is
 * contiguous. */
typedef struct mx_lowrank {
    const uint16_t* down; /* device BF16 [rank, K]: L_down transposed (row r = column r of L_down) */
    const uint16_t* up;   /* device BF16 [N, rank]: L_up transposed */
    int32_t rank;         /* 16, 32, 48 or 64 */
} mx_lowrank;

/* Version of this ABI (MX_ABI_VERSION). */
int mx_abi_version(void);

/* Human-readable name of a status code (static storage). */
const char* mx_status_string(int status);

/* Message describing the calling thread's last failing call ("" if none). */
const char* mx_last_error(void);

/*
 * mx_quantize - dynamic quantization of a BF16 matrix (rows x cols, leading dimension ld_x
 * elements) to `fmt`.
 *  MXFP4 / MXFP8: per 32 consecutive columns, scale byte = clamp(floor(log2 amax) - emax,
 *    -127, 127) + 127 (all-zero block: 0; a NaN/Inf in the block: 0xFF with codes 0); codes are
 *    RNE(|x| * 2^-exponent) on the element grid, saturating, with the sign of x.
 *  NVFP4: per 16 columns, block scale sb = E4M3_rne_sat(amax / (6 * global_scale)) and codes
 *    E2M1_rne_sat(|x| / (sb * global_scale)), each the exact real rounded once; sb = 0 gives
 *    zero magnitudes; a NaN/Inf in the block gives scale 0x7F (E4M3 NaN) and codes 0.
 *    global_scale (> 0, finite) is ignored for the MX formats.
 * layout MX_LAYOUT_ROW_MAJOR: codes device [rows, cols/2] (FP4) or [rows, cols] (FP8) bytes,
 *   scales device [rows, cols/G] bytes.
 * layout MX_LAYOUT_TILED (MX formats, cols % 128 == 0): codes and scales in the tiled layout,
 *   of mx_tiled_bytes sizes, 16-byte aligned; the padding rows are written with zeros.
 * Requires cols % G == 0, ld_x >= cols, x 16-byte aligned, ld_x % 8 == 0.
 */
mx_status mx_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int32_t fmt,
                      int32_t layout, float global_scale, void* codes, uint8_t* scales,
                      void* stream);

/* Byte sizes of the codes and the scales of a rows x cols matrix of format fmt in the tiled
 * layout (MX formats, cols % 128 == 0).  Host-side arithmetic only. */
mx_status mx_tiled_bytes(int64_t rows, int64_t cols, int32_t fmt, size_t* code_bytes,
                         size_t* scale_bytes);

/*
 * mx_relayout - copy a quantized matrix into the other layout: src and dst have the same fmt
 * (MXFP4 or MXFP8), rows and cols (cols % 128 == 0) and different layouts.  The bytes are only
 * moved, never re-encoded; a tiled destination gets zero padding rows.  Used to prepare a
 * weight once for the GEMM, or to read a tiled matrix back in the canonical layout.
 */
mx_status mx_relayout(const mx_qmatrix* src, const mx_qmatrix* dst, void* stream);

/*
 * mx_dequantize - the values a quantized matrix stands for.  The MXFP4 model cards
 * ("intel-ai/Wan2.2-I2V-A14B-Lightning-Diffusers-MXFP4-AutoRound", Quantization Details) store
 * FP4 E2M1 codes with one E8M0 (power-of-two) scale per 32 elements; the NVFP4 card
 * ("Wan2.2-T2V-A14B-Diffusers-NVFP4-AutoRound", Model Details) adds an FP8 E4M3 scale per 16
 * and an FP32 global scale per tensor.  BF16 values: y = code * 2^(scale - 127) for MX (exact),
 * y = bf16_rne(code * sb * global_scale) for NVFP4 (one rounding of the exact product).  A NaN
 * scale byte gives NaN.  y: device BF16, rows x cols with leading dimension ld_y >= cols.
 * Row-major matrices only (mx_relayout converts a tiled one).
 */
mx_status mx_dequantize(const mx_qmatrix* q, uint16_t* y, int64_t ld_y, void* stream);

/*
 * mx_absmax - largest |x| of a BF16 matrix, written as one float to device memory *amax
 * (NaN-free input expected).  Used to derive an NVFP4 tensor's global scale.
 */
mx_status mx_absmax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, float* amax,
                    void* stream);

/* NVFP4 global scale of a tensor with largest magnitude amax: fp32(amax / (6 * 448)), 1 for
 * amax = 0.  Host-side arithmetic only. */
float mx_nvfp4_global_scale(float amax);

/* Largest cols of mx_norm / mx_norm_quantize. */
#define MX_NORM_MAX_COLS 7680

/*
 * mx_norm_quantize - the producer of a quantized linear's input, fused with its quantizer.  The
 * MXFP4 model card ("intel-ai/Wan2.2-I2V-A14B-Lightning-Diffusers-MXFP4-AutoRound", Quantization
 * Details) keeps the norm and the modulation table in front of the quantized linears at higher
 * precision and quantizes the linears' activations dynamically.  Per row of the BF16 matrix x
 * (rows x cols, leading dimension ld_x), in fp32:
 *    h = LayerNorm(x) * gamma + beta,  then  h = h * (1 + scale) + shift
 * (LayerNorm: mean, biased variance, 1/sqrt(var + eps); gamma, beta, scale, shift are device
 * F32 [cols] vectors, each optional: NULL is the identity).  h is rounded to BF16 and that BF16
 * matrix is quantized to fmt (MXFP4 or MXFP8) exactly as mx_quantize would: codes and scales in
 * `layout` (row-major, or tiled with padding rows zero), ready for mx_linear_q.
 * Requires cols % 32 == 0 (cols % 128 for tiled), cols <= MX_NORM_MAX_COLS, eps finite > 0,
 * x 16-byte aligned with ld_x % 8 == 0, the vectors 4-byte aligned, codes aligned as for
 * mx_quantize.  Buffers are sized as for mx_quantize (mx_tiled_bytes for the tiled layout).
 */
mx_status mx_norm_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, float eps,
                           const float* gamma, const float* beta, const float* scale,
                           const float* shift, int32_t fmt, int32_t layout, void* codes,
                           uint8_t* scales, void* stream);

/* mx_norm - the same producer unfused: writes the BF16 h (rows x cols, leading dimension ld_y,
 * 16-byte aligned, ld_y % 8 == 0) that mx_norm_quantize quantizes. */
mx_status mx_norm(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, float eps,
                  const float* gamma, const float* beta, const float* scale, const float* shift,
                  uint16_t* y, int64_t ld_y, void* stream);

/* Microscaled attention: head dimension and keys per block. */
#define MX_ATTN_HEAD_DIM 128
#define MX_ATTN_KVB 64

/*
 * mx_quantize_vt - the V operand of mx_attention.  The FP4 attention backend of the MXFP4 Wan2.2
 * model cards ("intel-ai/Wan2.2-I2V-A14B-Lightning-Diffusers-MXFP4-AutoRound", attention backends
 * and Performance Profile) is read as attention in the formats of the linear layer; V's
 * 32-element MXFP8 (E4M3) groups run along the key axis, the axis its product with the
 * probabilities sums over, so V is stored transposed.  Input v: device BF16, BH heads of an
 * S x D matrix, element (b, s, d) at v[b * hs_v + s * ld_v + d] (a [BH, S, D] tensor has
 * ld_v = D, hs_v = S * D; one batch of a [S, H * D] projection has ld_v = H * D, hs_v = D).
 * Output, in blocks of MX_ATTN_KVB keys (Sp = S rounded up to MX_ATTN_KVB, keys past S quantized
 * as zeros): codes [BH, Sp / 64, D, 64] E4M3 bytes -- code (b, s, d) at
 * ((b * Sp / 64 + s / 64) * D + d) * 64 + s % 64 -- and scales [BH, Sp / 64, D, 2] E8M0, the
 * scale of keys 32 g..32 g + 31 of block s / 64 at ((b * Sp / 64 + s / 64) * D + d) * 2 + g % 2.
 * Each 32-key group is quantized as mx_quantize quantizes an MXFP8 row group (bit for bit the
 * same rule).  Requires D % 32 == 0, BH <= 65535, S <= 2^24, v 16-byte aligned with ld_v and
 * hs_v multiples of 8, codes 16-byte aligned.
 * Caller owns every buffer.
 */
mx_status mx_quantize_vt(const uint16_t* v, int64_t BH, int64_t S, int64_t D, int64_t ld_v,
                         int64_t hs_v, uint8_t* codes, uint8_t* scales, void* stream);

/*
 * mx_attention - softmax(softmax_scale * Q K^T) V per head, with Q and K in MXFP4 and V and the
 * probabilities in MXFP8 (same pages as mx_quantize_vt).  Queries and keys may come from
 * sequences of different lengths: S_q query rows and S_kv key / value rows per head (the DiT's
 * first attention layer has S_kv = S_q; its second, attn2 in the MXFP4 card's Quantization
 * Details, takes keys and values from the conditioning context).  Per block of MX_ATTN_KVB keys,
 * with c = softmax_scale * log2(e): s = c (q . k) (keys past S_kv masked), m' = max(m, block
 * max), alpha = 2^(m - m'), p = 2^(s - m'), l = alpha l + sum p, o = alpha o + Q_MX8(p) . V (p
 * quantized to MXFP8 in groups of 32 consecutive keys); out = o / l.  Scores and o accumulate in
 * FP32 on the scaled matrix cores.  Accuracy against the exact (fp64) evaluation of that
 * definition: within 2e-3 * sum p^ |v^| / l per element, plus the effect of probabilities whose
 * fp32 evaluation rounds to a neighbouring E4M3 value; the matrix core accumulates a block's FP8
 * products to about 1e-4 of their absolute sum rather than exactly in binary32.
 *  q_codes/q_scales: row-major MXFP4 (mx_quantize's output) of BH heads of S_q x
 *        MX_ATTN_HEAD_DIM, row (b, s) at element offset b * hs_q + s * ld_q: codes byte
 *        (b * hs_q + s * ld_q) / 2, scale byte (b * hs_q + s * ld_q) / 32.
 *  k_codes/k_scales: the same for S_kv key rows with ld_k, hs_k.  ld_q, hs_q, ld_k, hs_k are
 *        multiples of 128; codes 16-byte and scales 4-byte aligned.
 *  vt_codes/vt_scales: mx_quantize_vt's output for BH, S_kv, D (codes 16-byte, scales 4-byte
 *        aligned).
 *  out: device BF16 (MX_OUT_BF16, the RNE of the FP32 result) or FP32, element (b, s, d) at
 *        b * hs_o + s * ld_o + d (s < S_q); 16-byte aligned, ld_o and hs_o multiples of 8.
 * Requires D == MX_ATTN_HEAD_DIM, BH <= 65535, 0 <= S_q, S_kv <= 2^24 with
 * (S_kv + 64) * ld_k / 2 < 2^32, softmax_scale finite and > 0; S_kv == 0 with S_q > 0 is an
 * error (MX_ERR_SHAPE).  S_q == 0 does nothing.  Caller owns every buffer; nothing is allocated.
 */
mx_status mx_attention(const uint8_t* q_codes, const uint8_t* q_scales, int64_t ld_q, int64_t hs_q,
                       const uint8_t* k_codes, const uint8_t* k_scales, int64_t ld_k, int64_t hs_k,
                       const uint8_t* vt_codes, const uint8_t* vt_scales, int64_t BH, int64_t S_q,
                       int64_t S_kv, int64_t D, float softmax_scale, int32_t out_dtype, void* out,
                       int64_t ld_o, int64_t hs_o, void* stream);

/* Bytes of workspace mx_linear needs for an M x K activation in act_fmt: the activation is
 * quantized dynamically on every call ("intel-ai/Wan2.2-I2V-A14B-Lightning-Diffusers-MXFP4-AutoRound",
 * Quantization Details: act_dynamic, activations quantized to MXFP4 at run time), so its codes
 * and scales are staged here -- in the tiled layout for the MX formats when K % 128 == 0 -- plus
 * the BF16 M x rank input of the low-rank branch when rank > 0 ("Wan2.2 W4A8 SVDQuant - NVIDIA
 * (CUDA) artifacts", introduction).  Host-side arithmetic only; 0 for M <= 0. */
size_t mx_linear_workspace_bytes(int64_t M, int64_t K, int32_t act_fmt, int32_t rank);

/*
 * mx_linear - the quantized linear layer on a BF16 activation a (M x K, leading dimension ld_a):
 * quantize a dynamically to act_fmt (act_global_scale is the static NVFP4 activation global
 * scale), then y = dequant(a) . dequant(w)^T in fp32 accumulation, then the epilogue.  Sources:
 * the W4A4 layer of "intel-ai/Wan2.2-I2V-A14B-Lightning-Diffusers-MXFP4-AutoRound" (Model
 * Summary: an MXFP4 W4A4 linear kernel with a block-scaled matrix multiply; Quantization Details:
 * dynamic MXFP4 activations, MXFP4 weights, F16 biases); the NVFP4 variant of
 * "Wan2.2-T2V-A14B-Diffusers-NVFP4-AutoRound" (Model Details: real FP4 GEMMs, not an activation
 * quantize-dequantize emulation, dynamic block scales under a static activation global scale);
 * the W4A8 variant and its rank-32 BF16 branch of "Wan2.2 W4A8 SVDQuant - NVIDIA (CUDA)
 * artifacts" (introduction).
 * Supported (act_fmt, w->fmt): (MXFP4, MXFP4) W4A4; (MXFP8, MXFP4) W4A8; (MXFP8, MXFP8) W8A8
 * (K % 128 == 0); (NVFP4, NVFP4).
 *  bias: device FP16 [N] or NULL.
 *  lr:   low-rank branch or NULL (MX formats only); y += bf16_rne(a . lr->down) . lr->up,
 *        added before the bias.  With a branch, 31 * ld_a + K must be below 2^30 (a 32-row
 *        block of a spans less than 2 GiB), else MX_ERR_SHAPE.
 *  epilogue MX_EPI_BIAS / MX_EPI_BIAS_GELU: out is BF16 (out_dtype MX_OUT_BF16) or FP32
 *        (MX_OUT_F32), M x N with leading dimension ld_out elements.  The BF16 result is the
 *        RNE of the FP32 result.
 *  epilogue MX_EPI_BIAS_GELU_QUANT_MXFP4: h = gelu_tanh(acc + bias) in fp32 is quantized to
 *        MXFP4 with groups of 32 along N: out receives codes [M, N/2] and out_scales [M, N/32]
 *        (contiguous; ld_out must be N; out_dtype ignored).  Requires N % 32 == 0.
 *  epilogue MX_EPI_BIAS_GELU_QUANT_MXFP4_TILED: the same codes and scales as an M x N MXFP4
 *        matrix in the tiled layout (mx_tiled_bytes(M, N) sizes, padding rows zero), ready to be
 *        the activation of the next linear.  Requires MXFP4 activations, K % 128 == 0,
 *        N % 128 == 0, ld_out == N, out and out_scales 16-byte aligned.
 *  workspace: device, >= mx_linear_workspace_bytes(M, K, act_fmt, rank) bytes, 256-byte
 *        aligned; its contents on return are unspecified.
 * w: row-major, or tiled (MX formats): a weight prepared once with mx_relayout or quantized
 *        directly into the tiled layout is the fast GEMM operand.
 * Requires K % 32 == 0 (K % 16 == 0 for NVFP4, K % 128 == 0 for MXFP8 weights), w->cols == K,
 * N = w->rows >= 1.
 */
mx_status mx_linear(const uint16_t* a, int64_t M, int64_t K, int64_t ld_a, int32_t act_fmt,
                    float act_global_scale, const mx_qmatrix* w, const uint16_t* bias,
                    const mx_lowrank* lr, int32_t epilogue, int32_t out_dtype, void* out,
                    int64_t ld_out, uint8_t* out_scales, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Bytes of the static device workspace of mx_linear_noalloc (64 MiB per GPU). */
#define MX_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * mx_linear_noalloc - mx_linear for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  Same arguments, same
 * kernels and bit-identical results as mx_linear, without the workspace arguments: the
 * workspace is a statically allocated device array of MX_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, held from the first call on that GPU until the process ends.  It calls
 * no allocating routine.
 *  - Limit: mx_linear_workspace_bytes(M, K, act_fmt, rank) <= MX_NOALLOC_SCRATCH_BYTES, else
 *    MX_ERR_WORKSPACE before anything is launched (MXFP4 at K = 5120: M up to 24576 rows;
 *    larger activations are split along M by the caller, rows being independent).
 *  - The array of the calling thread's current device is used; `stream` must belong to that
 *    device.  The first call on a device looks the array's device address up once
 *    (hipGetSymbolAddress); a failure there is MX_ERR_HIP.
 *  - Every call on one GPU shares that GPU's array, which keeps the last call's contents (no
 *    call relies on it starting at zero).  Calls whose executions overlap on one GPU (several
 *    streams, or several host threads) race on it: serialise them, e.g. on one stream.
 */
mx_status mx_linear_noalloc(const uint16_t* a, int64_t M, int64_t K, int64_t ld_a, int32_t act_fmt,
                            float act_global_scale, const mx_qmatrix* w, const uint16_t* bias,
                            const mx_lowrank* lr, int32_t epilogue, int32_t out_dtype, void* out,
                            int64_t ld_out, uint8_t* out_scales, void* stream);

/*
 * mx_linear_q - the same GEMM and epilogues on an already quantized activation a (M x K), e.g.
 * the MXFP4 output of a MX_EPI_BIAS_GELU_QUANT_MXFP4 call feeding the next linear.  The
 * quantized linears of "intel-ai/Wan2.2-I2V-A14B-Lightning-Diffusers-MXFP4-AutoRound"
 * (Quantization Details, coverage list) include both layers of each block's feed-forward network,
 * ffn.net.0.proj and ffn.net.2; the second consumes the first's GELU output, which this library
 * re-quantizes in the first GEMM's epilogue (the pages do not say where that quantization
 * happens).  No workspace and no low-rank branch.  a and w may each be row-major or tiled (MX
 * formats).
 */
mx_status mx_linear_q(const mx_qmatrix* a, const mx_qmatrix* w, const uint16_t* bias,
                      int32_t epilogue, int32_t out_dtype, void* out, int64_t ld_out,
                      uint8_t* out_scales, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP_H */
