// Quantizer, dequantizer and absmax kernels for gfx950.
//
// MX quantization (MXFP4 model cards, Quantization Details: per-32 E8M0 scales, activations
// quantized dynamically; W4A8 SVDQuant page: dynamic MXFP8 activations), bit-level rules of OCP
// MX v1.0: shared exponent floor(log2 amax) - emax, RNE onto the element grid with saturation,
// sign kept.  NVFP4 (NVFP4 model card, Model Details): per-16 E4M3 block scales under an FP32
// global scale.
//
// The quantizers are HBM-bound (2 bytes read, 0.53 / 1.03 bytes written per element): every
// thread moves one 16-byte vector of 8 BF16 values, four (MX) or two (NVFP4) neighbouring lanes
// own one scale group and reduce its amax with DPP quad permutes, and the code bytes of a wave
// land in one contiguous span.  All arithmetic that decides a code is exact: BF16 magnitudes
// are ordered like their bit patterns (so amax is an integer max), the scale is an exponent
// field subtraction, q = |x| * 2^-e is an exact binary32 product (fp32 denormals are enabled),
// and the NVFP4 thresholds are exact fp64 products compared against binary32 values.
#include "mx_common.h"
#include "mx_internal.h"

namespace mxk {

typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------------------------
// MXFP4 / MXFP8
// ---------------------------------------------------------------------------------------------
// One thread's 8 elements of a 32-element group (the group's four threads are one DPP quad):
// the group's scale byte and the thread's codes, 4 bytes (E2M1, lo) or 8 bytes (E4M3, lo, hi).
// The element rounding is the gfx950 scaled conversion (V_CVT_SCALEF32_PK_FP4_BF16 /
// _PK_FP8_BF16), which rounds |x| / 2^e to nearest-even on the element grid and keeps the sign;
// it was checked exhaustively against that rule on every BF16 value and scale exponent
// (subnormals included).  Two differences from the rule are handled here: E4M3 overflow gives
// the NaN code instead of saturating, so magnitudes are first clamped to 448 * 2^e (they can
// exceed it only by less than one binade, q < 512); and a NaN/Inf in the group gives all-zero
// codes with scale 0xFF.
template <int ELEM>  // 0: E2M1 (emax 2), 1: E4M3 (emax 8)
__device__ __forceinline__ void quant_mx8(const uint4 v, uint32_t& lo, uint32_t& hi, uint32_t& sbyte) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
  u16x2 m2 = {0, 0};  // per-half maxima of the magnitudes (packed 16-bit max)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u16x2 mag;
    const uint32_t wm = w[i] & 0x7FFF7FFFu;
    __builtin_memcpy(&mag, &wm, 4);
    m2 = __builtin_elementwise_max(m2, mag);
  }
  uint32_t amax = max((uint32_t)m2.x, (uint32_t)m2.y);
  amax = max(amax, quad_xor1(amax));
  amax = max(amax, quad_xor2(amax));
  const bool bad = amax >= 0x7F80u;  // NaN or Inf in the group
  const int E = (int)(amax >> 7);    // BF16 exponent field of amax
  const int emax = ELEM == 0 ? 2 : 8;
  int e = E - 127 - emax;            // floor(log2 amax) - emax (subnormal/zero: clamped below)
  if (e < -127) e = -127;
  // 2^e as a binary32 (2^-127 is subnormal)
  const float scale = __uint_as_float(e >= -126 ? (uint32_t)(127 + e) << 23 : 0x00400000u);
  bf2v b[4];
  if (ELEM == 1) {
    const uint32_t lim = (uint32_t)((e + 135) << 7 | 0x60);  // BF16 bits of 448 * 2^e
    const u16x2 lim2 = {(uint16_t)lim, (uint16_t)lim};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u16x2 mag;
      const uint32_t m = w[i] & 0x7FFF7FFFu;
      __builtin_memcpy(&mag, &m, 4);
      mag = __builtin_elementwise_min(mag, lim2);
      uint32_t c;
      __builtin_memcpy(&c, &mag, 4);
      w[i] = c | (w[i] & 0x80008000u);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) __builtin_memcpy(&b[i], &w[i], 4);
  if (ELEM == 0) {
    uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, b[0], scale, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, b[1], scale, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, b[2], scale, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, b[3], scale, 3);
    lo = r;
    hi = 0;
  } else {
    i16x2 r0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(i16x2{0, 0}, b[0], scale, false);
    r0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r0, b[1], scale, true);
    i16x2 r1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(i16x2{0, 0}, b[2], scale, false);
    r1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r1, b[3], scale, true);
    __builtin_memcpy(&lo, &r0, 4);
    __builtin_memcpy(&hi, &r1, 4);
  }
  if (bad) lo = hi = 0;
  sbyte = bad ? 0xFFu : (uint32_t)(e + 127);
}

template <int ELEM>
__global__ void __launch_bounds__(256) quant_mx_kernel(const uint16_t* __restrict__ x,
                                                        int64_t rows, int64_t cols, int64_t ld,
                                                        uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales) {
  const int64_t gpr = cols >> 5;       // groups per row
  const int64_t total = rows * gpr * 4;  // four threads per group
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total; t += stride) {
    const int64_t g = t >> 2;
    const int part = (int)(t & 3);
    const int64_t r = g / gpr;
    const int64_t gc = g - r * gpr;
    uint32_t lo, hi, sbyte;
    quant_mx8<ELEM>(load_stream16(x + r * ld + gc * 32 + part * 8), lo, hi, sbyte);
    if (ELEM == 0) *(uint32_t*)(codes + r * (cols >> 1) + gc * 16 + part * 4) = lo;
    else *(uint2*)(codes + r * cols + gc * 32 + part * 8) = make_uint2(lo, hi);
    if (part == 0) scales[r * gpr + gc] = (uint8_t)sbyte;
  }
}

// Tiled output: a workgroup quantizes 16 rows x 512 columns per step (16 threads per row, four
// 128-column chunks of 8 elements each), so each row is read as 1 KB contiguous and each chunk
// is written as one 1 KB FP4 code tile (two FP8 tiles) and a quarter of a scale tile.  The four
// loads of a thread are issued before any is used.  Rows from `rows` to the padded count
// quantize zeros (zero codes, scale byte 0).
template <int ELEM>
__global__ void __launch_bounds__(256) quant_mx_tiled_kernel(const uint16_t* __restrict__ x,
                                                              int64_t rows, int64_t cols, int64_t ld,
                                                              uint8_t* __restrict__ codes,
                                                              uint8_t* __restrict__ scales) {
  constexpr int IT = 4;
  const int64_t nkc = cols >> 7;
  const int64_t nkg = (nkc + IT - 1) / IT;  // groups of IT chunks per row block
  const int64_t items = (tiled_rows(rows) >> 4) * nkg;
  const int rl = threadIdx.x >> 4, c8 = threadIdx.x & 15;
  const int g4 = c8 >> 2, part = c8 & 3;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int64_t rb = it / nkg, kg = it - rb * nkg;
    const int64_t r = rb * 16 + rl;
    uint4 v[IT];
#pragma unroll
    for (int u = 0; u < IT; ++u) {
      const int64_t kb = kg * IT + u;
      v[u] = r < rows && kb < nkc ? load_stream16(x + r * ld + kb * 128 + c8 * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < IT; ++u) {
      const int64_t kb = kg * IT + u;
      if (kb >= nkc) break;  // uniform: the last group of a row block may be partial
      uint32_t lo, hi, sbyte;
      quant_mx8<ELEM>(v[u], lo, hi, sbyte);
      if (ELEM == 0) {
        *(uint32_t*)(codes + tiled_fp4_off(r, kb, g4, nkc) + part * 4) = lo;
      } else {
        // the group's 32 bytes are pieces 2 g4 and 2 g4 + 1; this thread's 8 bytes are half a piece
        *(uint2*)(codes + tiled_fp8_off(r, kb, 2 * g4 + (part >> 1), nkc) + (part & 1) * 8) = make_uint2(lo, hi);
      }
      if (part == 0) scales[tiled_scale_off(r, kb, nkc) + g4] = (uint8_t)sbyte;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Producer-fused quantizer: LayerNorm (+ affine) and modulation, then the MX group quantizer
// ---------------------------------------------------------------------------------------------
// A workgroup of NW <= 8 waves handles 4 rows per step (two workgroups per compute unit overlap
// each other's loads and barriers).  Wave w owns CPW consecutive 128-column chunks; a lane holds
// 8 columns (8 (lane & 15) ..) of each chunk in row lane >> 4.
// Row sums, then sums of squared deviations (two passes over the registers), are reduced across
// the 16 lanes of a row and then across the waves through LDS in a fixed order, so every wave
// sees the same mean and rstd.  h = (x - mean) * rstd * A[c] + B[c], with A = gamma (1 + scale)
// and B = beta (1 + scale) + shift built once per workgroup in LDS, is rounded to BF16; the MX
// quantizer then codes that BF16 tensor exactly as the standalone quantizer would (same group
// routine).  OUT 0 writes the BF16 h instead (the unfused producer).  Padding rows of a tiled
// output get zero codes and zero scale bytes.
constexpr int NORM_ROWS = 4, NORM_WAVES = 8;  // rows per step (one per 16 lanes), waves

template <int ELEM, int OUT, int CPW>  // OUT 0: BF16 h, 1: codes row-major, 2: codes tiled
__global__ void __launch_bounds__(NORM_WAVES * 64, 2) norm_quant_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                          int64_t cols, int64_t ld, float eps,
                                                          const float* __restrict__ gamma,
                                                          const float* __restrict__ beta,
                                                          const float* __restrict__ scale,
                                                          const float* __restrict__ shift,
                                                          uint16_t* __restrict__ y, int64_t ld_y,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  extern __shared__ float norm_lds[];  // A[cols], B[cols], psum[waves][16 rows], psq[waves][16 rows]
  const int nw = (int)(blockDim.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  float* A = norm_lds;
  float* B = A + cols;
  float* psum = B + cols;
  float* psq = psum + NORM_WAVES * NORM_ROWS;
  for (int64_t c = threadIdx.x; c < cols; c += blockDim.x) {
    const float s1 = 1.0f + (scale ? scale[c] : 0.0f);
    A[c] = (gamma ? gamma[c] : 1.0f) * s1;
    B[c] = (beta ? beta[c] : 0.0f) * s1 + (shift ? shift[c] : 0.0f);
  }
  __syncthreads();

  const int64_t nkc = (cols + 127) >> 7;
  const int rsub = lane >> 4, cs = lane & 15;
  const int g4 = cs >> 2, part = cs & 3;
  const float inv_n = 1.0f / (float)cols;
  const int64_t nrb = (OUT == 2 ? tiled_rows(rows) : rows + NORM_ROWS - 1) / NORM_ROWS;
  // this lane's columns of each chunk (loop-invariant), whether they exist, and the byte offset
  // of its 16-byte piece from the step's first row (past the end of the buffer for a missing
  // column: the bounds-checked buffer load then reads zero)
  int64_t colv[CPW];
  bool colok[CPW];
  uint32_t loff[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    colv[c] = (int64_t)(wave * CPW + c) * 128 + cs * 8;
    colok[c] = colv[c] < cols;
    loff[c] = colok[c] ? (uint32_t)((rsub * ld + colv[c]) * 2) : 0x80000000u;
  }
  // the rows of step rb through a buffer descriptor that ends after the last valid element of
  // the step's last valid row, so rows past the matrix (and steps past the last) read zero with
  // no per-lane test; the next step's are loaded as soon as the current step's are unpacked, so
  // their latency overlaps this step's work
  auto fetch = [&](int64_t rb, uint4 (&dst)[CPW]) {
    const int64_t r0 = rb * NORM_ROWS;
    const int64_t vr = rb < nrb ? min((int64_t)NORM_ROWS, rows - r0) : 0;
    const auto rs = make_rsrc(vr > 0 ? x + r0 * ld : x, vr > 0 ? (uint32_t)(((vr - 1) * ld + cols) * 2) : 0u);
#pragma unroll
    for (int c = 0; c < CPW; ++c) dst[c] = load16(rs, loff[c]);
  };
  uint4 vn[CPW];
  fetch(blockIdx.x, vn);
  for (int64_t rb = blockIdx.x; rb < nrb; rb += gridDim.x) {
    const int64_t r = rb * NORM_ROWS + rsub;
    // unpack once: the three passes read the same fp32 values
    float xv[CPW][8];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const uint32_t w[4] = {vn[c].x, vn[c].y, vn[c].z, vn[c].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xv[c][2 * e] = __uint_as_float(w[e] << 16);
        xv[c][2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      }
    }
    fetch(rb + gridDim.x, vn);
    // pass 1: row sums (columns past cols read as zero)
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc += xv[c][2 * e] + xv[c][2 * e + 1];
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) acc += __shfl_xor(acc, m);
    if (cs == 0) psum[wave * NORM_ROWS + rsub] = acc;
    __syncthreads();
    float mean;
    {
      float t = 0.0f;
      for (int w = 0; w < nw; ++w) t += psum[w * NORM_ROWS + rsub];
      mean = t * inv_n;
    }
    // pass 2: sums of squared deviations over the valid columns
    acc = 0.0f;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      float q = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float d0 = xv[c][2 * e] - mean;
        const float d1 = xv[c][2 * e + 1] - mean;
        q += d0 * d0 + d1 * d1;
      }
      acc += colok[c] ? q : 0.0f;
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) acc += __shfl_xor(acc, m);
    if (cs == 0) psq[wave * NORM_ROWS + rsub] = acc;
    __syncthreads();
    float rstd;
    {
      float t = 0.0f;
      for (int w = 0; w < nw; ++w) t += psq[w * NORM_ROWS + rsub];
      rstd = __builtin_amdgcn_rsqf(t * inv_n + eps);
    }
    // pass 3: h, BF16, then the output
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int64_t kb = wave * CPW + c;
      if (kb >= nkc) break;  // uniform across the wave
      const int64_t col = colv[c];
      const bool valid = colok[c];
      float a[8], b[8];
      if (valid) {
        *(float4*)&a[0] = *(const float4*)&A[col];
        *(float4*)&a[4] = *(const float4*)&A[col + 4];
        *(float4*)&b[0] = *(const float4*)&B[col];
        *(float4*)&b[4] = *(const float4*)&B[col + 4];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = b[e] = 0.0f;
      }
      uint32_t hb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float h0 = (xv[c][2 * e] - mean) * rstd * a[2 * e] + b[2 * e];
        const float h1 = (xv[c][2 * e + 1] - mean) * rstd * a[2 * e + 1] + b[2 * e + 1];
        hb[e] = pack_bf16x2(h0, h1);
      }
      if constexpr (OUT == 0) {
        if (r < rows && valid) *(uint4*)(y + r * ld_y + col) = make_uint4(hb[0], hb[1], hb[2], hb[3]);
      } else {
        uint32_t lo, hi, sbyte;
        quant_mx8<ELEM>(make_uint4(hb[0], hb[1], hb[2], hb[3]), lo, hi, sbyte);
        if constexpr (OUT == 2) {
          if (r >= rows) lo = hi = sbyte = 0;  // padding rows of the tiled layout
          if (ELEM == 0) *(uint32_t*)(codes + tiled_fp4_off(r, kb, g4, nkc) + part * 4) = lo;
          else *(uint2*)(codes + tiled_fp8_off(r, kb, 2 * g4 + (part >> 1), nkc) + (part & 1) * 8) = make_uint2(lo, hi);
          if (part == 0) scales[tiled_scale_off(r, kb, nkc) + g4] = (uint8_t)sbyte;
        } else {
          if (r < rows && valid) {
            if (ELEM == 0) *(uint32_t*)(codes + r * (cols >> 1) + (col >> 1)) = lo;
            else *(uint2*)(codes + r * cols + col) = make_uint2(lo, hi);
            if (part == 0) scales[r * (cols >> 5) + (col >> 5)] = (uint8_t)sbyte;
          }
        }
      }
    }
  }
}

// Row-major <-> tiled copy: one thread per 16-byte code piece (and, for the first piece of each
// 128-column chunk, the row's 4 scale bytes of that chunk).  Padding rows of a tiled destination
// are zero-filled.
template <int ELEM, bool TO_TILED>
__global__ void __launch_bounds__(256) relayout_kernel(const uint8_t* __restrict__ sc, const uint8_t* __restrict__ ss,
                                                        uint8_t* __restrict__ dc, uint8_t* __restrict__ ds,
                                                        int64_t rows, int64_t cols) {
  const int64_t nkc = cols >> 7;
  constexpr int PPC = ELEM == 0 ? 4 : 8;  // 16-byte pieces per row and chunk
  const int64_t row_bytes = ELEM == 0 ? cols >> 1 : cols;
  const int64_t nrows = TO_TILED ? tiled_rows(rows) : rows;
  const int64_t total = nrows * nkc * PPC;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total; t += stride) {
    const int64_t r = t / (nkc * PPC);
    const int64_t j = t - r * (nkc * PPC);  // piece index within the row
    const int64_t kb = j / PPC;
    const int g = (int)(j - kb * PPC);
    const int64_t rm = r * row_bytes + j * 16;
    const int64_t ti = ELEM == 0 ? tiled_fp4_off(r, kb, g, nkc) : tiled_fp8_off(r, kb, g, nkc);
    const int64_t rs = r * (cols >> 5) + kb * 4, ts = tiled_scale_off(r, kb, nkc);
    if (TO_TILED) {
      const bool in = r < rows;
      *(uint4*)(dc + ti) = in ? *(const uint4*)(sc + rm) : make_uint4(0, 0, 0, 0);
      if (g == 0) *(uint32_t*)(ds + ts) = in ? *(const uint32_t*)(ss + rs) : 0u;
    } else {
      *(uint4*)(dc + rm) = *(const uint4*)(sc + ti);
      if (g == 0) *(uint32_t*)(ds + rs) = *(const uint32_t*)(ss + ts);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// NVFP4
// ---------------------------------------------------------------------------------------------
// binary32 value just below a positive finite one
__device__ __forceinline__ float prev_float(float f) { return __uint_as_float(__float_as_uint(f) - 1u); }

// Largest binary32 value <= t (t > 0 exact double).
__device__ __forceinline__ float f64_round_down(double t) {
  float f = (float)t;
  if ((double)f > t) f = prev_float(f);
  return f;
}

// Thresholds of the E2M1 rounding for block scale D = sb * sg, as binary32 values such that
// for a binary32 magnitude a:  code = sum_j [a > T_j].  The midpoints are 0.25, 0.75, 1.25,
// 1.75, 2.5, 3.5, 5; ties at 0.25, 1.25, 2.5, 5 round down (to the even code) and ties at 0.75,
// 1.75, 3.5 round up.  For a strict ">" against the exact t*D, any binary32 a satisfies
// a > t*D <=> a > RD(t*D).  For ">=", a >= t*D <=> a > prev(t*D) when t*D is a binary32 value,
// else <=> a > RD(t*D).
struct NvThresholds {
  float t[7];
};

__device__ __forceinline__ NvThresholds nv_thresholds(double D, bool zero) {
  NvThresholds th;
  const double mids[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
  const bool ge[7] = {false, true, false, true, false, true, false};
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    if (zero) {
      th.t[j] = __uint_as_float(0x7F800000u);  // +inf: every magnitude rounds to 0
      continue;
    }
    double T = mids[j] * D;  // exact: <= 3 + 28 significant bits
    float f = f64_round_down(T);
    if (ge[j] && (double)f == T) f = prev_float(f);
    th.t[j] = f;
  }
  return th;
}

// Positive binary32 q rounded to its nearest value with BITS significant bits (ties away; q is
// never a tie where this is used).
template <int BITS>
__device__ __forceinline__ float round_sig(float q) {
  constexpr uint32_t drop = 24 - BITS;
  return __uint_as_float((__float_as_uint(q) + (1u << (drop - 1))) & ~((1u << drop) - 1u));
}

// One thread per 16-element group (two 16-byte loads), NV_U groups per thread and step, all
// loaded before any is coded.  Every rounding below is exact; the fast paths are binary32
// brackets:
//  - Block scale sb = E4M3_rne_sat(amax / (6 sg)).  amax * (1/(6 sg)) in binary32 (product and
//    reciprocal each within an ulp) is within 2^-22 of the exact quotient, so nudging it by 2^-20
//    down and up brackets the quotient strictly; since RNE is monotone, equal E4M3 codes for the
//    two ends are the exact code.  Different codes are neighbours, and the quotient lies within
//    about 2^-19 of the E4M3 midpoint between them, which has at most 5 significant bits: rounding
//    the bracket's end to 5 bits recovers it exactly, and the sign of amax - (6 m) sg, one fused
//    multiply-add (6 m is exact, the fma rounds once, and the difference is far above the
//    underflow range for the 6 sg allowed here), says on which side the quotient lies; on the
//    midpoint itself the even code wins.  A global scale outside that range takes the fp64
//    quotient (one rounding: an 8-bit by 26-bit quotient never lands on a false E4M3 midpoint).
//  - Elements: code = RNE(x / D), D = sb * sg, by the hardware FP32 -> E2M1 conversion of the two
//    nudged products x * (1/D) * (1 -+ 2^-20).  Equal codes are the exact code.  An element whose
//    two codes differ sits within about 2^-19 of an E2M1 midpoint (at most 3 significant bits);
//    that midpoint m is recovered by rounding, and the sign of |x| - (m sb) sg (m sb exact, one
//    fma) picks the code, the even one on a tie.  Only those elements are visited, one at a time
//    per lane.  A block whose D lies outside [2^-70, 2^100] (an all-zero block, say) is coded
//    against exact fp64-derived thresholds instead.
constexpr int NV_U = 2;

// IDX: the group-index type, 32-bit when the group count allows (cheaper division)
template <typename IDX>
__global__ void __launch_bounds__(256) quant_nv_kernel(const uint16_t* __restrict__ x,
                                                        int64_t rows, int64_t cols, int64_t ld,
                                                        float sg, uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales) {
  const IDX gpr = (IDX)(cols >> 4);  // 16-element groups per row
  const IDX total = (IDX)rows * gpr;
  const double six_sg = 6.0 * (double)sg;
  constexpr float kLo = 1.0f - 0x1p-20f, kHi = 1.0f + 0x1p-20f;
  const float c6 = 6.0f * sg;
  const bool scale_fast = c6 >= 0x1p-80f && c6 <= 0x1p100f;
  const float inv6 = __builtin_amdgcn_rcpf(c6);
  const float inv6_lo = inv6 * kLo, inv6_hi = inv6 * kHi;
  for (IDX base = (IDX)blockIdx.x * 256 * NV_U; base < total; base += (IDX)gridDim.x * 256 * NV_U) {
    uint4 v[NV_U][2];
    IDX rr[NV_U], gc[NV_U];
#pragma unroll
    for (int u = 0; u < NV_U; ++u) {
      const IDX g = base + u * 256 + threadIdx.x;
      rr[u] = g / gpr;
      gc[u] = g - rr[u] * gpr;
      const uint16_t* src = x + (int64_t)rr[u] * ld + (int64_t)gc[u] * 16;
      v[u][0] = g < total ? load_stream16(src) : make_uint4(0, 0, 0, 0);
      v[u][1] = g < total ? load_stream16(src + 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < NV_U; ++u) {
      const IDX g = base + u * 256 + threadIdx.x;
      if (g >= total) continue;
      const uint32_t w[8] = {v[u][0].x, v[u][0].y, v[u][0].z, v[u][0].w,
                             v[u][1].x, v[u][1].y, v[u][1].z, v[u][1].w};
      u16x2 m2 = {0, 0};  // per-half maxima of the magnitudes (packed 16-bit max)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        u16x2 mag;
        const uint32_t wm = w[i] & 0x7FFF7FFFu;
        __builtin_memcpy(&mag, &wm, 4);
        m2 = __builtin_elementwise_max(m2, mag);
      }
      const uint32_t amax = max((uint32_t)m2.x, (uint32_t)m2.y);
      const bool bad = amax >= 0x7F80u;
      const float af = bf16_to_f32(amax);
      uint32_t sbyte;
      if (scale_fast) {
        const float ql = af * inv6_lo;
        sbyte = e4m3_code(ql);
        if (!bad && sbyte != e4m3_code(af * inv6_hi)) {
          const float e = __builtin_fmaf(-(round_sig<5>(ql) * 6.0f), sg, af);
          sbyte += (e > 0.0f || (e == 0.0f && (sbyte & 1u))) ? 1u : 0u;
        }
      } else {
        sbyte = e4m3_code_f64((double)af / six_sg);
      }
      // sbyte <= 126: a positive finite E4M3 value (normal ones: exponent field + 120 as the
      // binary32 exponent, the 3 mantissa bits on top of binary32's)
      const float sb = sbyte >= 8u ? __uint_as_float((sbyte << 20) + (120u << 23)) : (float)sbyte * 0x1p-9f;
      const float d32 = sb * sg;
      uint32_t out0 = 0, out1 = 0;
      if (d32 >= 0x1p-70f && d32 <= 0x1p100f) {
        const float inv = __builtin_amdgcn_rcpf(d32);
        const float il = inv * kLo, ih = inv * kHi;
        uint32_t hi0 = 0, hi1 = 0;
        static_for<4>([&](auto q) {
          constexpr int Q = decltype(q)::value;
          const float a0 = bf16_to_f32(w[Q] & 0xFFFFu), a1 = __uint_as_float(w[Q] & 0xFFFF0000u);
          const float b0 = bf16_to_f32(w[4 + Q] & 0xFFFFu), b1 = __uint_as_float(w[4 + Q] & 0xFFFF0000u);
          out0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out0, a0 * il, a1 * il, 1.0f, Q);
          hi0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi0, a0 * ih, a1 * ih, 1.0f, Q);
          out1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out1, b0 * il, b1 * il, 1.0f, Q);
          hi1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi1, b0 * ih, b1 * ih, 1.0f, Q);
        });
        // elements near a midpoint: nibbles where the two brackets disagree (out* holds the
        // lower magnitude, the upper one is one step above)
        uint32_t d0 = bad ? 0u : out0 ^ hi0, d1 = bad ? 0u : out1 ^ hi1;
        while (d0 | d1) {
          const bool first = d0 != 0u;
          const uint32_t nib = (uint32_t)__builtin_ctz(first ? d0 : d1) >> 2;
          const uint32_t el = nib + (first ? 0u : 8u);  // element index in the group
          const uint32_t wa = (el & 2u) ? ((el & 8u) ? w[5] : w[1]) : ((el & 8u) ? w[4] : w[0]);
          const uint32_t wb = (el & 2u) ? ((el & 8u) ? w[7] : w[3]) : ((el & 8u) ? w[6] : w[2]);
          const uint32_t word = (el & 4u) ? wb : wa;
          const float a = __uint_as_float(((el & 1u) ? word >> 16 : word) << 17 >> 1);
          const float e = __builtin_fmaf(-(round_sig<3>(a * il) * sb), sg, a);
          const uint32_t lo = ((first ? out0 : out1) >> (4 * nib)) & 7u;
          const uint32_t up = (e > 0.0f || (e == 0.0f && (lo & 1u))) ? 1u << (4 * nib) : 0u;
          const uint32_t clr = ~(0xFu << (4 * nib));
          if (first) {
            out0 += up;
            d0 &= clr;
          } else {
            out1 += up;
            d1 &= clr;
          }
        }
      } else {
        const NvThresholds th = nv_thresholds((double)sb * (double)sg, sbyte == 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t b = (w[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
          const float a = bf16_to_f32(b & 0x7FFFu);
          uint32_t c = 0;
#pragma unroll
          for (int j = 0; j < 7; ++j) c += a > th.t[j] ? 1u : 0u;
          c |= (b >> 12) & 8u;
          if (i < 8) out0 |= c << (4 * i);
          else out1 |= c << (4 * (i - 8));
        }
      }
      if (bad) out0 = out1 = 0;
      *(uint2*)(codes + (int64_t)rr[u] * (cols >> 1) + (int64_t)gc[u] * 8) = make_uint2(out0, out1);
      scales[(int64_t)rr[u] * gpr + (int64_t)gc[u]] = bad ? (uint8_t)0x7F : (uint8_t)sbyte;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// dequantization (one thread per 8 elements)
// ---------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) dequant_kernel(const uint8_t* __restrict__ codes,
                                                       const uint8_t* __restrict__ scales,
                                                       int64_t rows, int64_t cols, int fmt,
                                                       float sg, uint16_t* __restrict__ y,
                                                       int64_t ld) {
  const int64_t per_row = cols >> 3;
  const int64_t total = rows * per_row;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total; t += stride) {
    const int64_t r = t / per_row;
    const int64_t c0 = (t - r * per_row) * 8;
    uint32_t out[4];
    if (fmt == 1) {  // MXFP8
      const uint2 cb = *(const uint2*)(codes + r * cols + c0);
      const uint32_t s = scales[r * (cols >> 5) + (c0 >> 5)];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t code = ((i < 4 ? cb.x : cb.y) >> (8 * (i & 3))) & 0xFFu;
        float v = s == 0xFF ? __uint_as_float(0x7FC00000u)
                            : __builtin_amdgcn_ldexpf(e4m3_value(code), (int)s - 127);
        uint32_t h = f32_to_bf16_rne(v);
        out[i >> 1] = (i & 1) ? (out[i >> 1] | (h << 16)) : h;
      }
    } else {
      const uint32_t cb = *(const uint32_t*)(codes + r * (cols >> 1) + (c0 >> 1));
      if (fmt == 0) {  // MXFP4: exact
        const uint32_t s = scales[r * (cols >> 5) + (c0 >> 5)];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          uint32_t code = (cb >> (4 * i)) & 0xFu;
          float v = s == 0xFF ? __uint_as_float(0x7FC00000u)
                              : __builtin_amdgcn_ldexpf(e2m1_value(code), (int)s - 127);
          uint32_t h = f32_to_bf16_rne(v);
          out[i >> 1] = (i & 1) ? (out[i >> 1] | (h << 16)) : h;
        }
      } else {  // NVFP4: one rounding of code * sb * sg
        const uint32_t sbyte = scales[r * (cols >> 4) + (c0 >> 4)];
        const double sbg = (double)e4m3_value(sbyte) * (double)sg;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          uint32_t code = (cb >> (4 * i)) & 0xFu;
          uint32_t h = f64_to_bf16_rne((double)e2m1_value(code) * sbg);
          out[i >> 1] = (i & 1) ? (out[i >> 1] | (h << 16)) : h;
        }
      }
    }
    *(uint4*)(y + r * ld + c0) = make_uint4(out[0], out[1], out[2], out[3]);
  }
}

// ---------------------------------------------------------------------------------------------
// absmax: one workgroup, deterministic (max is order independent)
// ---------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) absmax_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                       int64_t cols, int64_t ld,
                                                       float* __restrict__ out) {
  __shared__ uint32_t red[1024];
  uint32_t m = 0;
  const int64_t total = rows * cols;
  for (int64_t i = threadIdx.x; i < total; i += 1024) {
    const int64_t r = i / cols;
    m = max(m, (uint32_t)(x[r * ld + (i - r * cols)] & 0x7FFFu));
  }
  red[threadIdx.x] = m;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] = max(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = bf16_to_f32(red[0]);
}

// ---------------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------------
static int grid_for(int64_t threads) {
  int64_t blocks = (threads + 255) / 256;
  const int64_t cap = 256 * 64;  // enough resident waves to cover HBM latency
  return (int)(blocks < cap ? (blocks > 0 ? blocks : 1) : cap);
}

hipError_t launch_quant_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int elem,
                           uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t threads = rows * (cols / 32) * 4;
  if (threads == 0) return hipSuccess;
  if (elem == 0)
    quant_mx_kernel<0><<<grid_for(threads), 256, 0, s>>>(x, rows, cols, ld, codes, scales);
  else
    quant_mx_kernel<1><<<grid_for(threads), 256, 0, s>>>(x, rows, cols, ld, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quant_mx_tiled(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int elem,
                                 uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t items = (tiled_rows(rows) / 16) * ((cols / 128 + 3) / 4);
  if (items == 0) return hipSuccess;
  const int grid = (int)(items < 256 * 32 ? items : 256 * 32);
  if (elem == 0)
    quant_mx_tiled_kernel<0><<<grid, 256, 0, s>>>(x, rows, cols, ld, codes, scales);
  else
    quant_mx_tiled_kernel<1><<<grid, 256, 0, s>>>(x, rows, cols, ld, codes, scales);
  return hipGetLastError();
}

hipError_t launch_relayout(const uint8_t* src_codes, const uint8_t* src_scales, uint8_t* dst_codes,
                           uint8_t* dst_scales, int64_t rows, int64_t cols, int elem, bool to_tiled,
                           hipStream_t s) {
  const int64_t nrows = to_tiled ? tiled_rows(rows) : rows;
  const int64_t threads = nrows * (cols / 128) * (elem == 0 ? 4 : 8);
  if (threads == 0) return hipSuccess;
  const int grid = grid_for(threads);
  if (elem == 0) {
    if (to_tiled) relayout_kernel<0, true><<<grid, 256, 0, s>>>(src_codes, src_scales, dst_codes, dst_scales, rows, cols);
    else relayout_kernel<0, false><<<grid, 256, 0, s>>>(src_codes, src_scales, dst_codes, dst_scales, rows, cols);
  } else {
    if (to_tiled) relayout_kernel<1, true><<<grid, 256, 0, s>>>(src_codes, src_scales, dst_codes, dst_scales, rows, cols);
    else relayout_kernel<1, false><<<grid, 256, 0, s>>>(src_codes, src_scales, dst_codes, dst_scales, rows, cols);
  }
  return hipGetLastError();
}

template <int ELEM, int OUT, int CPW>
static void run_norm(int grid, int threads, size_t lds, hipStream_t s, const uint16_t* x, int64_t rows,
                     int64_t cols, int64_t ld, float eps, const float* gamma, const float* beta,
                     const float* scale, const float* shift, uint16_t* y, int64_t ld_y,
                     uint8_t* codes, uint8_t* scales) {
  norm_quant_kernel<ELEM, OUT, CPW><<<grid, threads, lds, s>>>(x, rows, cols, ld, eps, gamma, beta, scale,
                                                               shift, y, ld_y, codes, scales);
}
template <int ELEM, int OUT>
static void run_norm_c(int cpw, int grid, int threads, size_t lds, hipStream_t s, const uint16_t* x,
                       int64_t rows, int64_t cols, int64_t ld, float eps, const float* gamma,
                       const float* beta, const float* scale, const float* shift, uint16_t* y,
                       int64_t ld_y, uint8_t* codes, uint8_t* scales) {
#define MX_NORM_CASE(C) \
  case C: run_norm<ELEM, OUT, C>(grid, threads, lds, s, x, rows, cols, ld, eps, gamma, beta, scale, shift, y, ld_y, codes, scales); break;
  switch (cpw) {
    MX_NORM_CASE(1) MX_NORM_CASE(2) MX_NORM_CASE(3) MX_NORM_CASE(4)
    MX_NORM_CASE(5) MX_NORM_CASE(6) MX_NORM_CASE(7) MX_NORM_CASE(8)
    default: break;
  }
#undef MX_NORM_CASE
}

hipError_t launch_norm_quant(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, float eps,
                             const float* gamma, const float* beta, const float* scale,
                             const float* shift, int out_kind, int elem, uint16_t* y, int64_t ld_y,
                             uint8_t* codes, uint8_t* scales, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int64_t nkc = (cols + 127) / 128;
  if (nkc > NORM_WAVES * 8) return hipErrorInvalidValue;
  // a step's four rows are addressed with 32-bit buffer offsets below 2^31
  if ((NORM_ROWS * ld + cols) * 2 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const int cpw = (int)((nkc + NORM_WAVES - 1) / NORM_WAVES);
  const int nw = (int)((nkc + cpw - 1) / cpw);
  const int threads = nw * 64;
  const size_t lds = (size_t)(2 * cols + 2 * NORM_WAVES * NORM_ROWS) * sizeof(float);
  const int64_t nrb = (out_kind == 2 ? tiled_rows(rows) : rows + NORM_ROWS - 1) / NORM_ROWS;
#ifndef MX_NORM_GRID
#define MX_NORM_GRID 512
#endif
  // persistent workgroups (two per compute unit): the A/B vectors are built once per workgroup
  const int grid = (int)(nrb < MX_NORM_GRID ? nrb : MX_NORM_GRID);
  if (out_kind == 0) run_norm_c<0, 0>(cpw, grid, threads, lds, s, x, rows, cols, ld, eps, gamma, beta, scale, shift, y, ld_y, codes, scales);
  else if (out_kind == 1 && elem == 0) run_norm_c<0, 1>(cpw, grid, threads, lds, s, x, rows, cols, ld, eps, gamma, beta, scale, shift, y, ld_y, codes, scales);
  else if (out_kind == 1) run_norm_c<1, 1>(cpw, grid, threads, lds, s, x, rows, cols, ld, eps, gamma, beta, scale, shift, y, ld_y, codes, scales);
  else if (elem == 0) run_norm_c<0, 2>(cpw, grid, threads, lds, s, x, rows, cols, ld, eps, gamma, beta, scale, shift, y, ld_y, codes, scales);
  else run_norm_c<1, 2>(cpw, grid, threads, lds, s, x, rows, cols, ld, eps, gamma, beta, scale, shift, y, ld_y, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quant_nv(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, float sg,
                           uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t groups = rows * (cols / 16);
  if (groups == 0) return hipSuccess;
  const int grid = grid_for((groups + NV_U - 1) / NV_U);
  // the 32-bit index must also hold the last step's base + the step without wrapping
  if (groups + (int64_t)grid * 256 * NV_U < ((int64_t)1 << 32))
    quant_nv_kernel<uint32_t><<<grid, 256, 0, s>>>(x, rows, cols, ld, sg, codes, scales);
  else
    quant_nv_kernel<int64_t><<<grid, 256, 0, s>>>(x, rows, cols, ld, sg, codes, scales);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                          int fmt, float sg, uint16_t* y, int64_t ld, hipStream_t s) {
  const int64_t threads = rows * (cols / 8);
  if (threads == 0) return hipSuccess;
  dequant_kernel<<<grid_for(threads), 256, 0, s>>>(codes, scales, rows, cols, fmt, sg, y, ld);
  return hipGetLastError();
}

hipError_t launch_absmax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, float* out,
                         hipStream_t s) {
  absmax_kernel<<<1, 1024, 0, s>>>(x, rows, cols, ld, out);
  return hipGetLastError();
}

}  // namespace mxk
