// Device-side helpers shared by the gfx950 kernels of this library (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mxk {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------------------------
// storage conversions
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// fp32 -> bf16, round to nearest even (NaN -> quiet NaN, overflow -> inf).
// Two binary32 values rounded to nearest-even BF16, packed lo | hi << 16: gfx950's
// V_CVT_PK_BF16_F32 (probed against the RNE rule on 8.4M values incl. ties, subnormals and
// overflow; a NaN stays a NaN).
typedef float v2f32 __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const v2bf16 r = __builtin_convertvector(v2f32{lo, hi}, v2bf16);
  uint32_t u;
  __builtin_memcpy(&u, &r, 4);
  return u;
}
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// fp64 -> bf16 with one rounding (nearest even) of the exact double value.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double v) {
  uint64_t u = (uint64_t)__double_as_longlong(v);
  uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
  uint64_t ua = u & 0x7FFFFFFFFFFFFFFFull;
  if (ua > 0x7FF0000000000000ull) return 0x7FC0u;  // NaN
  double a = __longlong_as_double((long long)ua);
  if (a < 0x1p-126) {  // BF16 subnormal range: quantum 2^-133 (result 128 = smallest normal)
    double m = __builtin_rint(a * 0x1p133);
    return sign | (uint32_t)m;
  }
  // keep 7 of the 52 stored mantissa bits, ties to even
  uint64_t r = (ua + 0xFFFFFFFFFFFull + ((ua >> 45) & 1ull)) >> 45;
  int64_t e = (int64_t)(r >> 7) - 1023 + 127;
  if (e >= 255) return sign | 0x7F80u;
  return sign | (uint32_t)((e << 7) | (int64_t)(r & 0x7F));
}

__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  const unsigned short hs = (unsigned short)h;
  _Float16 hv;
  __builtin_memcpy(&hv, &hs, 2);
  return (float)hv;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (read once, do not keep in cache)
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Raw buffer loads (gfx9 descriptor: no stride, bounds checked against num_records; an access
// past the end reads zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
  return make_uint2(v[0], v[1]);
}
// Direct-to-LDS buffer loads (CDNA4 "buffer_load_dword{,x4} ... lds"): lane i of the wave writes
// its 4 or 16 bytes at LDS address m0 + 4i / 16i.  Written as inline asm so that the compiler
// does not wait on them before unrelated LDS reads: the caller waits explicitly (vmcnt) before
// the barrier that publishes the chunk.  The asm has no register outputs; its VGPR/SGPR inputs
// are consumed at issue.  The descriptor is an SGPR quad (gfx9 raw buffer, num_records bounds
// check: accesses past the end read zero).
__device__ __forceinline__ v4i make_rsrc_sgpr(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  v4i r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}
__device__ __forceinline__ void dma_lds16(v4i rs, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds_addr), "v"(voff), "s"(rs), "s"(soff) : "memory", "m0");
}
__device__ __forceinline__ void dma_lds4(v4i rs, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(lds_addr), "v"(voff), "s"(rs), "s"(soff) : "memory", "m0");
}
// Wait for all vector-memory operations / all LDS operations of the wave.  Builtins, not asm,
// so that the compiler's own wait-count bookkeeping sees them (after vmcnt(0) it knows nothing
// of its own is in flight and inserts no further waits that would also stall on the DMA).
// Encodings (gfx9 s_waitcnt): vmcnt [3:0]+[15:14], expcnt [6:4], lgkmcnt [11:8].
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void wait_lds_all() { __builtin_amdgcn_s_waitcnt(0xC07F); }
template <typename T>
__device__ __forceinline__ uint32_t lds_addr_of(T* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)p;
}

__device__ __forceinline__ uint32_t load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t load2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t load1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}

// ---------------------------------------------------------------------------------------------
// element encodings (OCP MX v1.0).  Inputs are exact non-negative magnitudes.
// ---------------------------------------------------------------------------------------------
// E2M1 magnitude code of q, round to nearest even, saturating at 6.
//  q < 1: the grid is 0, 0.5 (step 0.5): code = rne(2q) in {0, 1, 2}.
//  q >= 1: one mantissa bit: round the binary32 pattern at bit 22, then the exponent and the
//  kept bit give the code directly (1.0 -> 2 ... 6.0 -> 7, 8.0 and above saturate to 7).
__device__ __forceinline__ uint32_t e2m1_code(float q) {
  if (q < 1.0f) return (uint32_t)__builtin_rintf(q * 2.0f);
  uint32_t u = __float_as_uint(q);
  uint32_t r = (u + 0x1FFFFFu + ((u >> 22) & 1u)) >> 22;
  uint32_t c = r - 252u;
  return c > 7u ? 7u : c;
}

// E4M3 magnitude code of q, round to nearest even, subnormal step 2^-9, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_code(float q) {
  if (q < 0.015625f) return (uint32_t)__builtin_rintf(q * 512.0f);
  uint32_t u = __float_as_uint(q);
  uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20;
  uint32_t c = r - (120u << 3);
  return c > 126u ? 126u : c;
}

// Same from an fp64 magnitude (one rounding of the double value).
__device__ __forceinline__ uint32_t e4m3_code_f64(double q) {
  if (q < 0.015625) return (uint32_t)__builtin_rint(q * 512.0);
  uint64_t u = (uint64_t)__double_as_longlong(q);
  uint64_t r = (u + 0xFFFFFFFFFFFFull + ((u >> 49) & 1ull)) >> 49;
  int64_t c = (int64_t)r - ((1023 - 7) << 3);
  return c > 126 ? 126u : (uint32_t)c;
}

// Decoded magnitudes.
__device__ __forceinline__ float e2m1_value(uint32_t code) {
  // 0, 0.5, 1, 1.5, 2, 3, 4, 6 as binary32 exponent/mantissa, sign from bit 3
  uint32_t m = code & 7u;
  uint32_t bits = m == 0 ? 0u : m == 1 ? 0x3F000000u : ((126u + (m >> 1)) << 23) | ((m & 1u) << 22);
  return __uint_as_float(bits | ((code & 8u) << 28));
}

__device__ __forceinline__ float e4m3_value(uint32_t b) {
  uint32_t e = (b >> 3) & 0xFu, m = b & 7u;
  float v;
  if (e == 0xF && m == 7) return __uint_as_float(0x7FC00000u);
  if (e == 0) v = (float)m * 0x1p-9f;
  else v = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (b & 0x80u) ? -v : v;
}

// ---------------------------------------------------------------------------------------------
// V_MFMA_SCALE_F32_32X32X64_F8F6F4 with operand vectors sized by format (the intrinsic is
// overloaded on them; the clang builtin only exposes the 8-dword form, which would keep four
// zero registers per FP4 operand).  The format, op_sel and scale-select arguments must be
// compile-time constants at the call site.
// ---------------------------------------------------------------------------------------------
__device__ v16f mfma_scale_32x32x64_f4f4(v4i a, v4i b, v16f c, int fmt_a, int fmt_b, int opsel_a,
                                         int scale_a, int opsel_b, int scale_b)
    __asm("llvm.amdgcn.mfma.scale.f32.32x32x64.f8f6f4.v4i32.v4i32");
__device__ v16f mfma_scale_32x32x64_f4f8(v4i a, v8i b, v16f c, int fmt_a, int fmt_b, int opsel_a,
                                         int scale_a, int opsel_b, int scale_b)
    __asm("llvm.amdgcn.mfma.scale.f32.32x32x64.f8f6f4.v4i32.v8i32");

// ---------------------------------------------------------------------------------------------
// one lane's 32-element MXFP8 group
// ---------------------------------------------------------------------------------------------
typedef __bf16 bf2x __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

// One lane's 32-element MXFP8 group (16 BF16 pairs): the same rule and instruction sequence as
// the standalone MX quantizer (amax, scale byte floor(log2 amax) - 8 clamped to [-127, 127],
// magnitudes clamped to 448 * 2^e because the conversion overflows to NaN instead of saturating,
// then V_CVT_SCALEF32_PK_FP8_BF16), with the amax taken within the lane.  NaN/Inf in the group:
// codes 0, scale byte 0xFF.
__device__ __forceinline__ void quant_fp8_group32(const uint32_t (&w)[16], uint32_t (&out)[8], uint32_t& sbyte) {
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = max(amax, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  const bool bad = amax >= 0x7F80u;
  int e = (int)(amax >> 7) - 127 - 8;
  if (e < -127) e = -127;
  const float scale = __uint_as_float(e >= -126 ? (uint32_t)(127 + e) << 23 : 0x00400000u);
  const uint32_t lim = (uint32_t)((e + 135) << 7 | 0x60);  // BF16 bits of 448 * 2^e
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    bf2x b[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t v = w[2 * q + k];
      const uint32_t lo = min(v & 0x7FFFu, lim), hi = min((v >> 16) & 0x7FFFu, lim);
      const uint32_t c = lo | (hi << 16) | (v & 0x80008000u);
      __builtin_memcpy(&b[k], &c, 4);
    }
    s16x2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(s16x2{0, 0}, b[0], scale, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, b[1], scale, true);
    uint32_t d;
    __builtin_memcpy(&d, &r, 4);
    out[q] = bad ? 0u : d;
  }
  sbyte = bad ? 0xFFu : (uint32_t)(e + 127);
}

// One lane's 32-element MXFP4 group (16 BF16 pairs), amax within the lane: the standalone MX
// quantizer's rule and instruction (scale byte floor(log2 amax) - 2 clamped to [-127, 127], then
// V_CVT_SCALEF32_PK_FP4_BF16).  out[d] byte j codes elements 8d + 2j and 8d + 2j + 1 (low
// nibble first), the FP4 operand layout.  NaN/Inf in the group: codes 0, scale byte 0xFF.
__device__ __forceinline__ void quant_fp4_group32(const uint32_t (&w)[16], uint32_t (&out)[4], uint32_t& sbyte) {
  typedef uint16_t u16x2g __attribute__((ext_vector_type(2)));
  u16x2g m2 = {0, 0};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    u16x2g mag;
    const uint32_t wm = w[i] & 0x7FFF7FFFu;
    __builtin_memcpy(&mag, &wm, 4);
    m2 = __builtin_elementwise_max(m2, mag);
  }
  const uint32_t amax = max((uint32_t)m2.x, (uint32_t)m2.y);
  const bool bad = amax >= 0x7F80u;
  int e = (int)(amax >> 7) - 127 - 2;
  if (e < -127) e = -127;
  const float scale = __uint_as_float(e >= -126 ? (uint32_t)(127 + e) << 23 : 0x00400000u);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    bf2x b[4];
    __builtin_memcpy(b, &w[4 * d], 16);
    uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, b[0], scale, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, b[1], scale, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, b[2], scale, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, b[3], scale, 3);
    out[d] = bad ? 0u : r;
  }
  sbyte = bad ? 0xFFu : (uint32_t)(e + 127);
}

// ---------------------------------------------------------------------------------------------
// cross-lane helpers
// ---------------------------------------------------------------------------------------------
// max with the lane xor 1 / xor 2 inside each quad (DPP quad_perm)
__device__ __forceinline__ uint32_t quad_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
}
__device__ __forceinline__ uint32_t quad_xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
}

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// Compile-time loop: f(std::integral_constant<int, I>) for I = 0 .. N-1.  Register arrays indexed
// through it always see constant indices, whatever the unroller decides for large bodies.
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// Tiled GEMM operand layout (MX formats, columns a multiple of 128, rows padded to 256): the
// byte offsets of one 16-byte code piece and of one row's 4 scale bytes of a 128-column chunk.
constexpr int TILE_ROWS = 256;
__host__ __device__ inline int64_t tiled_rows(int64_t rows) { return (rows + TILE_ROWS - 1) / TILE_ROWS * TILE_ROWS; }
// FP4: 1 KB tile = 16 rows x 128 columns; piece g (0..3) of row r in chunk kb
__device__ __forceinline__ int64_t tiled_fp4_off(int64_t r, int64_t kb, int g, int64_t nkc) {
  return ((r >> 4) * nkc + kb) * 1024 + (r & 15) * 64 + ((g ^ (int)((r >> 2) & 3)) << 4);
}
// FP8: 1 KB tile = 8 rows x 128 columns; piece g (0..7) of row r in chunk kb
__device__ __forceinline__ int64_t tiled_fp8_off(int64_t r, int64_t kb, int g, int64_t nkc) {
  return ((r >> 3) * nkc + kb) * 1024 + (r & 7) * 128 + ((g ^ (int)((r >> 1) & 7)) << 4);
}
// scales: 256-byte tile = 64 rows x 4 bytes
__device__ __forceinline__ int64_t tiled_scale_off(int64_t r, int64_t kb, int64_t nkc) {
  return ((r >> 6) * nkc + kb) * 256 + (r & 63) * 4;
}

}  // namespace mxk
