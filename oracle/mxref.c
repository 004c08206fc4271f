/*
 * CPU ORACLE for the microscaled-FP4 linear layer and the microscaled attention.  TEST INFRASTRUCTURE ONLY: nothing in the
 * product library links, includes or calls this file; only the tests, the smoke check and the
 * CPU-baseline leg of the benchmark do.  It shares no code, header or table with the HIP path.
 *
 * Plain, slow and exact: every floating-point value is held in fp64, every rounding is written
 * out once from its definition, OpenMP only splits independent rows.
 *
 * Sources (model cards of quantized Wan2.2 transformers):
 *  - "Wan2.2-I2V-A14B-Lightning-Diffusers-MXFP4-AutoRound", Quantization Details: MXFP4 W4A4,
 *    weights packed as FP4 E2M1 two per byte with one E8M0 scale per 32 elements, activations
 *    quantized dynamically at run time, group size 32, symmetric, F16 biases.
 *  - "Wan2.2-Animate-14B-Diffusers-MXFP4-AutoRound", Quantization Details: same format (RTN).
 *  - "Wan2.2-T2V-A14B-Diffusers-NVFP4-AutoRound", Model Details: NVFP4 = E2M1 elements, group
 *    16, FP8 E4M3 block scales, FP32 global scales; block scales dynamic, global activation
 *    scale static (calibrated).
 *  - "Wan2.2 W4A8 SVDQuant - NVIDIA (CUDA) artifacts": MXFP4 weights x dynamic MXFP8
 *    activations + a rank-32 low-rank correction with BF16 factors.
 *  - "Wan2.2-I2V-A14B-Lightning-Diffusers-MXFP4-AutoRound", Quantization Details, list of layers
 *    kept at higher precision (norm, modulation table): the LayerNorm + modulation that produces
 *    a quantized linear's input (mxr_norm_modulate).
 *  - "Wan2.2-I2V-A14B-Lightning-Diffusers-MXFP4-AutoRound", attention backends and Performance
 *    Profile, and "Wan2.2-Animate-14B-Diffusers-MXFP4-AutoRound" on the FP4 attention backend:
 *    microscaled attention in the formats of the linear layer (mxr_attention_mx).
 * The pages name these formats but do not define them bit by bit; the element and scale
 * encodings follow the OCP Microscaling (MX) v1.0 specification that the "MX" names refer to.
 * Where the pages are silent, each function below states the reading it takes.
 *
 * Parity status: every function here is pinned by a CPU test against values the pages fix, a
 * hand-derived worked example, a brute-force search, exact rational arithmetic or a library
 * routine (the tests of the oracle name the pin of each function).  The NVFP4 global scale
 * other than 1 is pinned by hand-derived blocks, an exact rational brute force of the quantizer,
 * the decode as an exact product and a rational brute-force GEMM; the attention's probability
 * quantization, its 32-key grouping, its flip bound and its absolute accumulator are pinned by a
 * constructed case whose scores are exact.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------------------------------ */
/* Storage types                                                                              */
/* ------------------------------------------------------------------------------------------ */

/* BF16 bit pattern -> exact value (BF16 is the top half of an IEEE binary32). */
double mxr_bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* FP16 (IEEE binary16) bit pattern -> exact value. */
double mxr_f16_value(uint16_t h) {
    int s = h >> 15, e = (h >> 10) & 0x1F, m = h & 0x3FF;
    double v;
    if (e == 0x1F) v = m ? NAN : INFINITY;
    else if (e == 0) v = ldexp((double)m, -24);
    else v = ldexp((double)(1024 + m), e - 25);
    return s ? -v : v;
}

/* Round a real (held exactly in fp64) to BF16, round-to-nearest-even, overflow to infinity.
 * Written directly from the definition (8 significant bits, exponent range of binary32) rather
 * than through a binary32 intermediate, so there is exactly one rounding. */
uint16_t mxr_bf16_rne(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | 0x7F80;
    int ex;
    frexp(a, &ex);                 /* a = f * 2^ex, f in [0.5, 1): floor(log2 a) = ex - 1 */
    int e = ex - 1;
    if (e < -126) e = -126;        /* subnormal quantum 2^-133 */
    double quantum = ldexp(1.0, e - 7);
    double n = a / quantum;        /* exact: division by a power of two */
    double r = floor(n);
    double frac = n - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
    double rv = r * quantum;       /* exactly representable in BF16 (or 2^128 on overflow) */
    if (rv >= 0x1.0p128) return sign | 0x7F80;
    float f = (float)rv;           /* exact */
    uint32_t u;
    memcpy(&u, &f, 4);
    return sign | (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------------------------------ */
/* Element and scale formats (OCP MX v1.0)                                                    */
/* ------------------------------------------------------------------------------------------ */

/* FP4 E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit, no Inf/NaN.  The eight
 * magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double mxr_e2m1_value(unsigned code) {
    unsigned s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, (int)e - 1);
    return s ? -v : v;
}

/* FP8 E4M3 (OCP "E4M3", no infinities): sign, 4 exponent bits (bias 7), 3 mantissa bits;
 * S.1111.111 is NaN, the largest finite magnitude is 448 = 1.75 * 2^8. */
double mxr_e4m3_value(unsigned byte) {
    unsigned s = (byte >> 7) & 1, e = (byte >> 3) & 0xF, m = byte & 7;
    double v;
    if (e == 0xF && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp(1.0 + m / 8.0, (int)e - 7);
    return s ? -v : v;
}

/* E8M0 scale: 2^(byte - 127); 0xFF is NaN. */
double mxr_e8m0_value(unsigned byte) {
    if (byte == 0xFF) return NAN;
    return ldexp(1.0, (int)byte - 127);
}

/* RNE of a non-negative exact real q onto the E2M1 magnitudes, ties to the code with an even
 * least significant bit, saturating at 6 (E2M1 has no infinity).  Walks the grid pairwise. */
unsigned mxr_e2m1_rne_mag(double q) {
    for (unsigned c = 0; c < 7; ++c) {
        double lo = mxr_e2m1_value(c), hi = mxr_e2m1_value(c + 1);
        if (q <= hi) {
            double mid = 0.5 * (lo + hi);
            if (q < mid) return c;
            if (q > mid) return c + 1;
            return (c % 2 == 0) ? c : c + 1;
        }
    }
    return 7; /* q > 6: saturate */
}

/* RNE of a non-negative exact real q onto the E4M3 magnitudes (subnormals kept), saturating at
 * 448 and never producing the NaN encoding.  Returns the 7-bit magnitude code. */
unsigned mxr_e4m3_rne_mag(double q) {
    if (q == 0.0) return 0;
    int ex;
    frexp(q, &ex);
    int e = ex - 1;               /* floor(log2 q) */
    if (e < -6) e = -6;           /* subnormal binade shares the quantum 2^-9 */
    double quantum = ldexp(1.0, e - 3);
    double n = q / quantum;       /* exact */
    double r = floor(n);
    double frac = n - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
    double v = r * quantum;
    if (v > 448.0) v = 448.0;
    /* encode the representable magnitude v */
    if (v < ldexp(1.0, -6)) return (unsigned)(v / ldexp(1.0, -9)); /* subnormal: m * 2^-9 */
    frexp(v, &ex);
    int ve = ex - 1;
    unsigned m = (unsigned)((v / ldexp(1.0, ve) - 1.0) * 8.0);
    return (unsigned)((ve + 7) << 3) | m;
}

/* ------------------------------------------------------------------------------------------ */
/* MX block quantization                                                                      */
/* ------------------------------------------------------------------------------------------ */

enum { MXR_E2M1 = 0, MXR_E4M3 = 1 };

/* Quantize one block of n reals (n = 32 for MX) to element codes (sign included, unpacked) and
 * one E8M0 scale byte.
 *  1. A NaN or infinity anywhere in the block: scale 0xFF (E8M0 NaN), codes 0.
 *  2. amax = max |x_i|.  The shared exponent is floor(log2 amax) - emax_elem, with emax 2 for
 *     E2M1 and 8 for E4M3 (OCP MX v1.0); amax = 0 gives -127.  Clamped to [-127, 127];
 *     the scale byte is exponent + 127.
 *  3. q_i = |x_i| * 2^-exponent (exact), rounded to nearest-even onto the element grid with
 *     saturation at the largest magnitude; the sign bit is x_i's sign bit (so -0 and negative
 *     values that round to zero keep it). */
void mxr_mx_block(const double* x, int n, int elem, unsigned char* codes, unsigned char* scale) {
    const int emax = (elem == MXR_E2M1) ? 2 : 8;
    double amax = 0.0;
    for (int i = 0; i < n; ++i) {
        if (!isfinite(x[i])) {
            *scale = 0xFF;
            for (int j = 0; j < n; ++j) codes[j] = 0;
            return;
        }
        if (fabs(x[i]) > amax) amax = fabs(x[i]);
    }
    int e;
    if (amax == 0.0) {
        e = -127;
    } else {
        int ex;
        frexp(amax, &ex);
        e = (ex - 1) - emax;
    }
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    *scale = (unsigned char)(e + 127);
    for (int i = 0; i < n; ++i) {
        double q = ldexp(fabs(x[i]), -e);
        unsigned s = signbit(x[i]) ? 1u : 0u;
        if (elem == MXR_E2M1) codes[i] = (unsigned char)((s << 3) | mxr_e2m1_rne_mag(q));
        else codes[i] = (unsigned char)((s << 7) | mxr_e4m3_rne_mag(q));
    }
}

/* Pack E2M1 codes two per byte: element 2j in the low nibble, 2j+1 in the high nibble. */
static void pack_e2m1(const unsigned char* c, int n, uint8_t* out) {
    for (int j = 0; j < n / 2; ++j) out[j] = (uint8_t)((c[2 * j] & 0xF) | ((c[2 * j + 1] & 0xF) << 4));
}

/* Quantize a row-major matrix (rows x cols, leading dimension ld, values held as fp64) to MX.
 * Groups are 32 consecutive columns starting at column 0 (cols % 32 == 0 is required).
 * Output: codes row-major [rows, cols/2] bytes (E2M1, packed) or [rows, cols] bytes (E4M3);
 * scales row-major [rows, cols/32].  Returns 0, or -1 on a shape error. */
int mxr_quantize_mx_f64(const double* x, int64_t rows, int64_t cols, int64_t ld, int elem,
                        uint8_t* codes, uint8_t* scales) {
    if (cols % 32) return -1;
    const int64_t groups = cols / 32;
    const int64_t code_row = (elem == MXR_E2M1) ? cols / 2 : cols;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        unsigned char c[32];
        for (int64_t g = 0; g < groups; ++g) {
            mxr_mx_block(x + r * ld + g * 32, 32, elem, c, scales + r * groups + g);
            if (elem == MXR_E2M1) pack_e2m1(c, 32, codes + r * code_row + g * 16);
            else memcpy(codes + r * code_row + g * 32, c, 32);
        }
    }
    return 0;
}

/* Same, from BF16 bit patterns (converted exactly to fp64 first). */
int mxr_quantize_mx_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int elem,
                         uint8_t* codes, uint8_t* scales) {
    if (cols % 32) return -1;
    const int64_t groups = cols / 32;
    const int64_t code_row = (elem == MXR_E2M1) ? cols / 2 : cols;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double v[32];
        unsigned char c[32];
        for (int64_t g = 0; g < groups; ++g) {
            for (int i = 0; i < 32; ++i) v[i] = mxr_bf16_value(x[r * ld + g * 32 + i]);
            mxr_mx_block(v, 32, elem, c, scales + r * groups + g);
            if (elem == MXR_E2M1) pack_e2m1(c, 32, codes + r * code_row + g * 16);
            else memcpy(codes + r * code_row + g * 32, c, 32);
        }
    }
    return 0;
}

/* Same, from fp32 values (for re-quantizing an fp32 intermediate). */
int mxr_quantize_mx_f32(const float* x, int64_t rows, int64_t cols, int64_t ld, int elem,
                        uint8_t* codes, uint8_t* scales) {
    if (cols % 32) return -1;
    const int64_t groups = cols / 32;
    const int64_t code_row = (elem == MXR_E2M1) ? cols / 2 : cols;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double v[32];
        unsigned char c[32];
        for (int64_t g = 0; g < groups; ++g) {
            for (int i = 0; i < 32; ++i) v[i] = (double)x[r * ld + g * 32 + i];
            mxr_mx_block(v, 32, elem, c, scales + r * groups + g);
            if (elem == MXR_E2M1) pack_e2m1(c, 32, codes + r * code_row + g * 16);
            else memcpy(codes + r * code_row + g * 32, c, 32);
        }
    }
    return 0;
}

/* Exact MX dequantization to fp64: value(code) * 2^(scale - 127) (NaN for scale 0xFF). */
void mxr_dequantize_mx(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                       int elem, double* out) {
    const int64_t groups = cols / 32;
    const int64_t code_row = (elem == MXR_E2M1) ? cols / 2 : cols;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < cols; ++c) {
            unsigned code;
            if (elem == MXR_E2M1) {
                uint8_t b = codes[r * code_row + c / 2];
                code = (c % 2 == 0) ? (b & 0xF) : (b >> 4);
            } else {
                code = codes[r * code_row + c];
            }
            double v = (elem == MXR_E2M1) ? mxr_e2m1_value(code) : mxr_e4m3_value(code);
            out[r * cols + c] = v * mxr_e8m0_value(scales[r * groups + c / 32]);
        }
    }
}

/* ------------------------------------------------------------------------------------------ */
/* NVFP4                                                                                      */
/* ------------------------------------------------------------------------------------------ */

/* Global scale of a tensor, stored in the decode direction: fp32_rne(amax / (6 * 448)), so that
 * the tensor's largest magnitude maps to the largest E2M1 value times the largest E4M3 block
 * scale.  amax = 0 gives 1.  (The page fixes only that a FP32 global scale exists; the
 * direction and the 6 * 448 normaliser are the reading used throughout.) */
float mxr_nv_global_scale(double amax) {
    if (amax == 0.0 || !isfinite(amax)) return 1.0f;
    /* amax (a BF16 value) and 2688 are exact binary32 values, so one binary32 division is the
     * exact quotient rounded once, to nearest-even */
    volatile float num = (float)amax, den = 2688.0f;
    return num / den;
}

/* Quantize one block of n (= 16) reals with decode-direction global scale sg.
 *  1. NaN/Inf in the block: scale byte 0x7F (E4M3 NaN), codes 0.
 *  2. sb = E4M3_rne_sat(amax / (6 * sg)), one rounding of the exact quotient.
 *  3. sb = 0: every magnitude is 0, signs kept.
 *  4. q_i = |x_i| / (sb * sg), one rounding to E2M1 (RNE, saturating at 6), sign kept.
 * fp64 suffices for "exact, then round once": the operands carry at most 8, 24 and 4
 * significant bits, so a quotient that is not a rounding midpoint lies at least ~2^-31
 * (relative) from every E4M3/E2M1 midpoint, far outside fp64's 2^-53 rounding error, and an
 * exact midpoint is computed exactly. */
void mxr_nv_block(const double* x, int n, float sg, unsigned char* codes, unsigned char* scale) {
    double amax = 0.0;
    for (int i = 0; i < n; ++i) {
        if (!isfinite(x[i])) {
            *scale = 0x7F;
            for (int j = 0; j < n; ++j) codes[j] = 0;
            return;
        }
        if (fabs(x[i]) > amax) amax = fabs(x[i]);
    }
    double g = (double)sg;
    unsigned sbyte = mxr_e4m3_rne_mag(amax / (6.0 * g));
    *scale = (unsigned char)sbyte;
    double sb = mxr_e4m3_value(sbyte);
    for (int i = 0; i < n; ++i) {
        unsigned s = signbit(x[i]) ? 1u : 0u;
        unsigned mag = (sb == 0.0) ? 0u : mxr_e2m1_rne_mag(fabs(x[i]) / (sb * g));
        codes[i] = (unsigned char)((s << 3) | mag);
    }
}

/* NVFP4 quantization of a BF16 matrix: codes [rows, cols/2] packed like MXFP4, E4M3 scales
 * [rows, cols/16].  cols % 16 == 0 is required. */
int mxr_quantize_nv_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, float sg,
                         uint8_t* codes, uint8_t* scales) {
    if (cols % 16) return -1;
    const int64_t groups = cols / 16;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double v[16];
        unsigned char c[16];
        for (int64_t g = 0; g < groups; ++g) {
            for (int i = 0; i < 16; ++i) v[i] = mxr_bf16_value(x[r * ld + g * 16 + i]);
            mxr_nv_block(v, 16, sg, c, scales + r * groups + g);
            pack_e2m1(c, 16, codes + r * (cols / 2) + g * 8);
        }
    }
    return 0;
}

/* Exact NVFP4 dequantization to fp64: value(code) * sb * sg (the product of 2-, 4- and
 * 24-significant-bit factors is exact in fp64). */
void mxr_dequantize_nv(const uint8_t* codes, const uint8_t* scales, float sg, int64_t rows,
                       int64_t cols, double* out) {
    const int64_t groups = cols / 16;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < cols; ++c) {
            uint8_t b = codes[r * (cols / 2) + c / 2];
            unsigned code = (c % 2 == 0) ? (b & 0xF) : (b >> 4);
            out[r * cols + c] = mxr_e2m1_value(code) * mxr_e4m3_value(scales[r * groups + c / 16]) *
                                (double)sg;
        }
    }
}

/* ------------------------------------------------------------------------------------------ */
/* Linear layer                                                                               */
/* ------------------------------------------------------------------------------------------ */

/* y[m, n] = sum_k a[m, k] * w[n, k] + bias[n]   (a: M x K, w: N x K, both dequantized, fp64)
 * abs_sum[m, n] = sum_k |a[m, k] * w[n, k]|     (the scale of the tolerance)
 * bias may be NULL; abs_sum may be NULL. */
void mxr_gemm_f64(const double* a, int64_t M, const double* w, int64_t N, int64_t K,
                  const double* bias, double* y, double* abs_sum) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        const double* ar = a + m * K;
        for (int64_t n = 0; n < N; ++n) {
            const double* wr = w + n * K;
            double s = 0.0, t = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = ar[k] * wr[k];
                s += p;
                t += fabs(p);
            }
            y[m * N + n] = s + (bias ? bias[n] : 0.0);
            if (abs_sum) abs_sum[m * N + n] = t;
        }
    }
}

/* tanh-form GELU, 0.5 y (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3))), in fp64 with the host libm
 * tanh (Hendrycks and Gimpel, "Gaussian Error Linear Units", the tanh approximation). */
double mxr_gelu_tanh(double y) {
    const double c = 0.79788456080286535587989211986876; /* sqrt(2/pi) */
    return 0.5 * y * (1.0 + tanh(c * (y + 0.044715 * y * y * y)));
}

void mxr_gelu_tanh_array(const double* y, int64_t n, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = mxr_gelu_tanh(y[i]);
}

/* Low-rank branch of SVDQuant: u[m, r] = bf16_rne(sum_k x[m, k] * down[k, r]) with x the
 * unquantized BF16 activation and down the BF16 K x R factor; then
 * y[m, n] += sum_r u[m, r] * up[r, n] with up the BF16 R x N factor.
 * lr[m, n] receives the low-rank term and lr_abs[m, n] = sum_r |u[m, r] up[r, n]|. */
void mxr_lowrank(const uint16_t* x, int64_t ldx, int64_t M, int64_t K, const uint16_t* down,
                 int64_t R, const uint16_t* up, int64_t N, uint16_t* u_out, double* lr,
                 double* lr_abs) {
    if (R > 256) return;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        double u[256];
        for (int64_t r = 0; r < R; ++r) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k)
                s += mxr_bf16_value(x[m * ldx + k]) * mxr_bf16_value(down[k * R + r]);
            uint16_t ub = mxr_bf16_rne(s);
            if (u_out) u_out[m * R + r] = ub;
            u[r] = mxr_bf16_value(ub);
        }
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0, t = 0.0;
            for (int64_t r = 0; r < R; ++r) {
                double p = u[r] * mxr_bf16_value(up[r * N + n]);
                s += p;
                t += fabs(p);
            }
            lr[m * N + n] = s;
            if (lr_abs) lr_abs[m * N + n] = t;
        }
    }
}

/* Largest |x| over a BF16 matrix (NaN-free input). */
double mxr_absmax_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld) {
    double amax = 0.0;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            double v = fabs(mxr_bf16_value(x[r * ld + c]));
            if (v > amax) amax = v;
        }
    return amax;
}

/* Element-wise BF16 rounding of an array of exact reals (see mxr_bf16_rne). */
void mxr_bf16_rne_array(const double* v, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = mxr_bf16_rne(v[i]);
}

/* ------------------------------------------------------------------------------------------ */
/* The layer in front of a quantized linear: LayerNorm and modulation                         */
/* ------------------------------------------------------------------------------------------ */
/* "Wan2.2-I2V-A14B-Lightning-Diffusers-MXFP4-AutoRound", Quantization Details: the quantized
 * linears quantize their activations dynamically, and the layers kept at higher precision in
 * front of them include the norm and the modulation table (F32).  The pages do not write these
 * layers out.  This is the textbook LayerNorm of a row (mean, biased variance, eps inside the
 * square root), an optional per-column affine y * gamma + beta, then the optional per-column
 * modulation y * (1 + scale) + shift.  fp64 throughout, from the exact BF16 / F32 inputs; a NULL
 * vector is the identity (gamma 1, beta 0, scale 0, shift 0).  h is [rows, cols], contiguous. */
void mxr_norm_modulate(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, double eps,
                       const float* gamma, const float* beta, const float* scale,
                       const float* shift, double* h) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * ld;
        double mean = 0.0;
        for (int64_t k = 0; k < cols; ++k) mean += mxr_bf16_value(xr[k]);
        mean /= (double)cols;
        double var = 0.0;
        for (int64_t k = 0; k < cols; ++k) {
            double d = mxr_bf16_value(xr[k]) - mean;
            var += d * d;
        }
        var /= (double)cols;
        double rstd = 1.0 / sqrt(var + eps);
        for (int64_t k = 0; k < cols; ++k) {
            double y = (mxr_bf16_value(xr[k]) - mean) * rstd;
            y = y * (gamma ? (double)gamma[k] : 1.0) + (beta ? (double)beta[k] : 0.0);
            y = y * (1.0 + (scale ? (double)scale[k] : 0.0)) + (shift ? (double)shift[k] : 0.0);
            h[r * cols + k] = y;
        }
    }
}

/* ------------------------------------------------------------------------------------------ */
/* Microscaled attention                                                                      */
/* ------------------------------------------------------------------------------------------ */
/* "intel-ai/Wan2.2-I2V-A14B-Lightning-Diffusers-MXFP4-AutoRound", attention backends and
 * Performance Profile: attention takes the larger share of the DiT's kernel time, and one of the
 * backends runs it as microscaled FP4 attention; "Wan2.2-Animate-14B-Diffusers-MXFP4-AutoRound"
 * notes that backend's lower fidelity.  The pages do not give its algorithm.  This is the reading
 * used here: blocked attention with an online softmax, in the formats of the linear layer.
 *  - Q and K rows (length D) are MXFP4 along D (the activation quantizer); V is MXFP8 (E4M3)
 *    along the key axis: Q_MX8 of V transposed, keys padded with zeros to whole blocks.
 *  - Per block of kvb keys: s_j = c * (q . k_j), c = softmax_scale * log2(e), keys past S
 *    masked; m' = max(m, max_j s_j); alpha = 2^(m - m'); p_j = 2^(s_j - m');
 *    l = alpha l + sum_j p_j; p^ = Q_MX8(p) in groups of 32 keys; o = alpha o + sum_j p^_j v^_j.
 *  - out = o / l.
 * fp64 throughout.  Queries and keys may come from sequences of different lengths: S query rows
 * and Skv key / value rows per head (self-attention has Skv = S; the DiT's second attention
 * layer, attn2 in the MXFP4 card's Quantization Details, takes its keys and values from the
 * conditioning context).  Only the query rows listed in qrows (indices into the BH*S rows) are
 * computed.  bound accumulates like o with the worst case of |p^_j - p_j| between two
 * implementations whose p differ by rounding noise: 2^(floor(log2 p_j) - 2) (a rounding step of
 * p, or the block scale moving across a power of two) plus the subnormal quantum 2^(e - 9), times
 * |v^_jd|; absacc accumulates sum_j p^_j |v^_jd|.  Both are divided by l like o. */
void mxr_attention_mx(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                      const uint8_t* vc, const uint8_t* vs, int64_t BH, int64_t S, int64_t Skv,
                      int64_t D, int64_t Sp, int kvb, double softmax_scale, const int64_t* qrows,
                      int64_t nq, double* out, double* bound, double* absacc) {
    (void)BH;
    const double c = softmax_scale / log(2.0);
#pragma omp parallel for schedule(dynamic)
    for (int64_t t = 0; t < nq; ++t) {
        const int64_t row = qrows[t], bh = row / S;
        double q[1024], o[1024], bnd[1024], ab[1024], s[256], p[256], ph[256], step[256];
        for (int64_t d = 0; d < D; ++d) {
            q[d] = mxr_e2m1_value((qc[row * (D / 2) + d / 2] >> (4 * (d & 1))) & 15) *
                   mxr_e8m0_value(qs[row * (D / 32) + d / 32]);
            o[d] = bnd[d] = ab[d] = 0.0;
        }
        double m = -INFINITY, l = 0.0;
        for (int64_t b0 = 0; b0 < Sp; b0 += kvb) {
            double mb = -INFINITY;
            for (int j = 0; j < kvb; ++j) {
                const int64_t key = b0 + j;
                if (key >= Skv) { s[j] = -INFINITY; continue; }
                const int64_t krow = bh * Skv + key;
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    dot += q[d] * mxr_e2m1_value((kc[krow * (D / 2) + d / 2] >> (4 * (d & 1))) & 15) *
                           mxr_e8m0_value(ks[krow * (D / 32) + d / 32]);
                s[j] = c * dot;
                if (s[j] > mb) mb = s[j];
            }
            const double mn = mb > m ? mb : m;
            const double alpha = (m == -INFINITY) ? 0.0 : exp2(m - mn);
            double psum = 0.0;
            for (int j = 0; j < kvb; ++j) {
                p[j] = (s[j] == -INFINITY) ? 0.0 : exp2(s[j] - mn);
                psum += p[j];
            }
            l = l * alpha + psum;
            for (int g = 0; g < kvb / 32; ++g) {
                unsigned char codes[32], sc;
                mxr_mx_block(p + 32 * g, 32, MXR_E4M3, codes, &sc);
                const double e = mxr_e8m0_value(sc);
                for (int j = 0; j < 32; ++j) {
                    const double pj = p[32 * g + j];
                    ph[32 * g + j] = mxr_e4m3_value(codes[j]) * e;
                    step[32 * g + j] = pj > 0.0 ? ldexp(1.0, ilogb(pj) - 2) + e * ldexp(1.0, -9) : 0.0;
                }
            }
            for (int64_t d = 0; d < D; ++d) {
                double acc = 0.0, accb = 0.0, acca = 0.0;
                for (int j = 0; j < kvb; ++j) {
                    const int64_t key = b0 + j;
                    const double v = mxr_e4m3_value(vc[(bh * D + d) * Sp + key]) *
                                     mxr_e8m0_value(vs[(bh * D + d) * (Sp / 32) + key / 32]);
                    acc += ph[j] * v;
                    accb += step[j] * fabs(v);
                    acca += ph[j] * fabs(v);
                }
                o[d] = o[d] * alpha + acc;
                bnd[d] = bnd[d] * alpha + accb;
                ab[d] = ab[d] * alpha + acca;
            }
            m = mn;
        }
        for (int64_t d = 0; d < D; ++d) {
            out[t * D + d] = o[d] / l;
            bound[t * D + d] = bnd[d] / l;
            absacc[t * D + d] = ab[d] / l;
        }
    }
}
