// Block-scaled GEMMs for gfx950 with fused epilogues.
//
// MXFP4 W4A4 (MXFP4 model cards, Quantization Details) and MXFP8 x MXFP4 W4A8 (W4A8 SVDQuant
// page) run on the CDNA4 scaled MFMA V_MFMA_SCALE_F32_32X32X64_F8F6F4: its K of 64 is two
// 32-element scale blocks, each lane supplies one E8M0 byte per operand and the bytes of the
// lanes of half b scale block b, so the per-32 MX scales cost nothing.  The MFMA "A" operand is
// the weight tile (n rows), the "B" operand the activation tile (m rows), which puts 16 values
// of one output row m, 4 consecutive n at a time, in each lane: the epilogue can store them as
// vectors and reduce a 32-wide re-quantization group with a single cross-lane exchange.
//
// The MX kernels share those conventions:
//  - the ring kernel (K % 128 == 0, every configuration of the model): an LDS ring of
//    128-element K chunks filled by direct-to-LDS buffer loads, operands row-major or in the
//    tiled layout whose 1 KB / 256 B tiles are exactly the LDS images the ring holds.  W4A4 on
//    a grid of at least 256 tiles runs 256 x 256 tiles, one workgroup of 8 waves per compute
//    unit in a ping-pong schedule (one wave per SIMD multiplies while the other loads); smaller
//    W4A4 grids and the low-rank branch run 256 x 128 tiles, W4A8 128 x 128 and W8A8 128 x 256,
//    two workgroups (one for W8A8) per compute unit;
//  - the register-staged kernel for any other K (a multiple of 32): 256-element chunks
//    double-buffered through registers, partial last chunk zero-filled;
//  - for W4A4 linears on a grid of a few tiles, one kernel that quantizes the BF16 activation
//    into LDS and multiplies (linear_fused_small_kernel), with the ring kernels' MFMA order.
// Sums over k are order-free, so each kernel pairs K blocks into MFMA steps in whatever order
// makes the per-lane scale bytes one op_sel-selected register (see each kernel).
//
// NVFP4 (NVFP4 model card, Model Details) has E4M3 scales per 16 elements that the scaled MFMA
// cannot apply, and code * scale needs up to 6 significant bits, more than FP8 holds; it is
// dequantized exactly after staging, to FP16 in the ring kernel (V_MFMA_F32_32X32X16_F16) and to
// BF16 in the register-staged one (V_MFMA_F32_32X32X16_BF16), with the product of the two FP32
// global scales applied in the epilogue.
#include "mx_common.h"
#include "mx_internal.h"

#include <stdlib.h>

namespace mxk {

constexpr int KC = 256;  // K elements per staged chunk

// Band heights (tile rows) of the XCD-ordered tile walks: the ring kernels (8) and the
// ping-pong W4A4 kernel (4: its 32 tiles per XCD span 4 rows of A and 8 columns of W).
#ifndef MX_RING_GM
#define MX_RING_GM 8
#endif
#ifndef MX_PP_GM
#define MX_PP_GM 4
#endif

// tanh-form GELU, 0.5 y (1 + tanh(u)) with u = sqrt(2/pi) (y + 0.044715 y^3), evaluated as the
// equal y / (1 + exp(-2u)): no cancellation for large negative y, and one hardware exp2 and one
// reciprocal (about 1 ulp each, a few 1e-7 relative overall; exp2 overflow gives the limit 0).
__device__ __forceinline__ float gelu_tanh_f32(float y) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  const float u = c * (y + 0.044715f * y * y * y);
  const float e = __builtin_amdgcn_exp2f(u * -2.8853900817779268f);  // exp(-2u) = 2^(-2u log2 e)
  return y * __builtin_amdgcn_rcpf(1.0f + e);
}

// Byte offset of 16-byte chunk c of LDS row `row` (rows of `rowb` = 128 or 256 bytes).  The
// chunk index is XORed with a function of the row so that the 16-byte reads of 16 consecutive
// rows at one chunk index (one quarter wave of ds_read_b128) land in 16 distinct 16-byte bank
// groups: for 128-byte rows two rows share a 256-byte bank window, so rows of one parity must
// differ in the XOR term, hence (row ^ row >> 3) & 7; 256-byte rows use row & 15.
__device__ __forceinline__ int swz(int row, int c, int rowb) {
  const int f = rowb == 128 ? ((row ^ (row >> 3)) & 7) : (row & 15);
  return row * rowb + ((c ^ f) << 4);
}

// XCD-aware tile order.  Workgroup b runs on XCD b % 8, each XCD with its own L2: give XCD x a
// contiguous range of tile indices, walked in bands of 4 tile rows (m) column by column, so
// that the ~32 tiles an XCD runs at once share 4 activation row-tiles and ~8 weight tiles.
__device__ __forceinline__ void tile_coords(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int q = total >> 3, r = total & 7;
  const int x = b & 7, j = b >> 3;
  const int t = x * q + min(x, r) + j;
  constexpr int GM = 4;
  const int band = t / (GM * tiles_n);
  const int in = t - band * GM * tiles_n;
  const int rows = min(GM, tiles_m - band * GM);
  tm = band * GM + in % rows;
  tn = in / rows;
}

// ---------------------------------------------------------------------------------------------
// epilogue: one 32 (n) x 32 (m) accumulator block
// ---------------------------------------------------------------------------------------------
// lane l holds m = mb + (l & 31) and n = nb + 8a + 4h + i for a, i in 0..3 (h = l >> 5):
// acc[4a + i].
// Bias of one 32-column block: the 16 values at this lane's n positions (zero without bias).
__device__ __forceinline__ void load_bias16(const GemmParams& p, int nb, float (&b)[16]) {
  const int h = lane_id() >> 5;
  // buffer loads: columns past N (and a missing bias) read as zero, without branches
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.bias, p.bias ? (uint32_t)p.N * 2u : 0u);
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const uint32_t off = (uint32_t)(nb + 8 * a + 4 * h) * 2u;
    if ((p.N & 3) == 0) {  // whole runs of 4 in or out of range
      const uint2 u = load8(rb, off);
      b[4 * a + 0] = f16_to_f32(u.x & 0xFFFFu);
      b[4 * a + 1] = f16_to_f32(u.x >> 16);
      b[4 * a + 2] = f16_to_f32(u.y & 0xFFFFu);
      b[4 * a + 3] = f16_to_f32(u.y >> 16);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) b[4 * a + i] = f16_to_f32(load2(rb, off + 2u * i));
    }
  }
}

// acc * out_scale + bias (fp32, after accumulation), then GELU for the GELU epilogues.
template <int EPI>
__device__ __forceinline__ void finish16(const GemmParams& p, const v16f& acc, const float (&b)[16],
                                         float (&v)[16]) {
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    v[e] = acc[e] * p.out_scale + b[e];
    if (EPI != EPI_BIAS) v[e] = gelu_tanh_f32(v[e]);
  }
}

// Direct stores of one block: lane l holds row m = mb + (l & 31), columns nb + 8a + 4h + i.
template <bool OUTF32>
__device__ __forceinline__ void store_block(const GemmParams& p, const float (&v)[16], int nb, int mb) {
  const int lane = lane_id();
  const int h = lane >> 5;
  const int m = mb + (lane & 31);
  if (m >= p.M) return;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int n = nb + 8 * a + 4 * h;
    if (OUTF32) {
      float* o = (float*)p.out + (int64_t)m * p.ld_out + n;
      if (n + 3 < p.N) {
        *(float4*)o = make_float4(v[4 * a], v[4 * a + 1], v[4 * a + 2], v[4 * a + 3]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (n + i < p.N) o[i] = v[4 * a + i];
      }
    } else {
      uint16_t* o = (uint16_t*)p.out + (int64_t)m * p.ld_out + n;
      const uint32_t p01 = pack_bf16x2(v[4 * a], v[4 * a + 1]), p23 = pack_bf16x2(v[4 * a + 2], v[4 * a + 3]);
      if (n + 3 < p.N) {
        *(uint2*)o = make_uint2(p01, p23);
      } else {
        const uint32_t bb[4] = {p01 & 0xFFFFu, p01 >> 16, p23 & 0xFFFFu, p23 >> 16};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (n + i < p.N) o[i] = (uint16_t)bb[i];
      }
    }
  }
}

// MXFP4 re-quantization of h along n: the 32 values of a block for row m live in lanes l and
// l ^ 32.  Same rule as the activation quantizer, on binary32 values: the element rounding is
// gfx950's V_CVT_SCALEF32_PK_FP4_F32 (|h| / 2^e to nearest-even on the E2M1 grid, sign kept;
// probed against that rule on 8.4M values incl. ties, their neighbours and subnormals).
// Requires N % 32 == 0.  TILED: codes and scales go to the tiled layout, and rows past M (up to
// the 256-row padding, which the tile covers) are written as zeros.
template <bool TILED>
__device__ __forceinline__ void requant_block(const GemmParams& p, const float (&v)[16], int nb, int mb) {
  const int lane = lane_id();
  const int h = lane >> 5;
  const int m = mb + (lane & 31);
  uint32_t amax = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) amax = max(amax, __float_as_uint(v[e]) & 0x7FFFFFFFu);
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 32));
  const bool bad = amax >= 0x7F800000u;
  int ex = (int)(amax >> 23) - 129;  // floor(log2 amax) - 2, clamped below
  if (ex < -127) ex = -127;
  const float scale = __uint_as_float(ex >= -126 ? (uint32_t)(127 + ex) << 23 : 0x00400000u);  // 2^ex
  uint32_t run[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[4 * a], v[4 * a + 1], scale, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[4 * a + 2], v[4 * a + 3], scale, 1);
    run[a] = bad ? 0u : (r & 0xFFFFu);  // 4 codes = 2 bytes at byte offset 4a + 2h of the block
  }
  const uint32_t X = run[0] | (run[1] << 16), Y = run[2] | (run[3] << 16);
  const uint32_t recv = (uint32_t)__shfl_xor((int)(h ? X : Y), 32);
  uint32_t d0, d1;
  if (h == 0) {  // bytes 0..7: own runs 0,1 (low halves) and the partner's runs 0,1
    d0 = (X & 0xFFFFu) | (recv << 16);
    d1 = (X >> 16) | (recv & 0xFFFF0000u);
  } else {       // bytes 8..15: partner's runs 2,3 and own runs 2,3 (high halves)
    d0 = (recv & 0xFFFFu) | (Y << 16);
    d1 = (recv >> 16) | (Y & 0xFFFF0000u);
  }
  uint8_t sbyte = bad ? (uint8_t)0xFF : (uint8_t)(ex + 127);
  uint8_t* codes = (uint8_t*)p.out;
  if (TILED) {
    if (nb < p.N) {
      if (m >= p.M) d0 = d1 = 0, sbyte = 0;  // padding rows
      const int64_t nkc = p.N >> 7, kb = nb >> 7;
      const int g = (nb & 127) >> 5;
      *(uint2*)(codes + tiled_fp4_off(m, kb, g, nkc) + 8 * h) = make_uint2(d0, d1);
      if (h == 0) p.out_scales[tiled_scale_off(m, kb, nkc) + g] = sbyte;
    }
  } else if (m < p.M && nb < p.N) {
    *(uint2*)(codes + (int64_t)m * (p.N >> 1) + (nb >> 1) + 8 * h) = make_uint2(d0, d1);
    if (h == 0) p.out_scales[(int64_t)m * (p.N >> 5) + (nb >> 5)] = sbyte;
  }
}

// One block through the compile-time epilogue.
template <int EPI, bool OUTF32>
__device__ __forceinline__ void epilogue_block_t(const GemmParams& p, const v16f& acc, const float (&b)[16],
                                                 int nb, int mb) {
  float v[16];
  finish16<EPI>(p, acc, b, v);
  if (EPI == EPI_GELU_QUANT || EPI == EPI_GELU_QUANT_T) requant_block<EPI == EPI_GELU_QUANT_T>(p, v, nb, mb);
  else store_block<OUTF32>(p, v, nb, mb);
}

// Run-time dispatch for the kernels that are not specialised by epilogue.
__device__ __forceinline__ void epilogue_block(const GemmParams& p, v16f acc, int nb, int mb) {
  float b[16];
  load_bias16(p, nb, b);
  if (p.epi == EPI_GELU_QUANT) epilogue_block_t<EPI_GELU_QUANT, false>(p, acc, b, nb, mb);
  else if (p.epi == EPI_GELU) {
    if (p.out_f32) epilogue_block_t<EPI_GELU, true>(p, acc, b, nb, mb);
    else epilogue_block_t<EPI_GELU, false>(p, acc, b, nb, mb);
  } else {
    if (p.out_f32) epilogue_block_t<EPI_BIAS, true>(p, acc, b, nb, mb);
    else epilogue_block_t<EPI_BIAS, false>(p, acc, b, nb, mb);
  }
}

// Direct epilogue of a wave's sub-tile (re-quantizing epilogue, or unaligned outputs).
template <int FN, int FM, int EPI, bool OUTF32>
__device__ __forceinline__ void epilogue_direct(const GemmParams& p, v16f (&acc)[FN][FM], int n_base,
                                                int m_base) {
  static_for<FN>([&](auto i) {
    const int nb = n_base + 32 * i;
    if (nb < p.N) {
      float b[16];
      load_bias16(p, nb, b);
      static_for<FM>([&](auto j) {
        __builtin_amdgcn_sched_barrier(0);  // one block at a time: keep register use small
        const int mb = m_base + 32 * j;
        if (mb < p.M || EPI == EPI_GELU_QUANT_T) epilogue_block_t<EPI, OUTF32>(p, acc[i][j], b, nb, mb);
      });
    }
  });
}

// low-rank term: acc += up_t[n, :] . u[m, :] over rank R (BF16 MFMA 32x32x16)
__device__ __forceinline__ v16f lowrank_block(const GemmParams& p, v16f acc, int nb, int mb) {
  const int lane = lane_id();
  const int h = lane >> 5;
  const int n = min(nb + (lane & 31), p.N - 1);
  const int m = min(mb + (lane & 31), p.M - 1);
  for (int r0 = 0; r0 < p.R; r0 += 16) {
    const uint4 wa = *(const uint4*)(p.lr_up + (int64_t)n * p.R + r0 + 8 * h);
    const uint4 ub = *(const uint4*)(p.lr_u + (int64_t)m * p.R + r0 + 8 * h);
    v8bf fa, fb;
    __builtin_memcpy(&fa, &wa, 16);
    __builtin_memcpy(&fb, &ub, 16);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc, 0, 0, 0);
  }
  return acc;
}

// The low-rank term of a wave's FN x FM blocks, in 16-rank slices [Q0, Q1): the fragments of
// up_t and u are loaded (lowrank_load, all in flight together), then the MFMAs (lowrank_mma).
// A kernel may load the first slices before its K loop, so that their latency is hidden.
template <int FN, int FM, int NQ>
struct LrFrags {
  uint4 wa[FN][NQ], ub[FM][NQ];
};
template <int FN, int FM, int Q0, int Q1>
__device__ __forceinline__ void lowrank_load(const GemmParams& p, LrFrags<FN, FM, Q1 - Q0>& f, int n_base, int m_base) {
  const int lane = lane_id();
  const int h = lane >> 5;
#pragma unroll
  for (int i = 0; i < FN; ++i) {
    const int n = min(n_base + 32 * i + (lane & 31), p.N - 1);
#pragma unroll
    for (int q = Q0; q < Q1; ++q)
      f.wa[i][q - Q0] = 16 * q < p.R ? *(const uint4*)(p.lr_up + (int64_t)n * p.R + 16 * q + 8 * h) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int m = min(m_base + 32 * j + (lane & 31), p.M - 1);
#pragma unroll
    for (int q = Q0; q < Q1; ++q)
      f.ub[j][q - Q0] = 16 * q < p.R ? *(const uint4*)(p.lr_u + (int64_t)m * p.R + 16 * q + 8 * h) : make_uint4(0, 0, 0, 0);
  }
}
template <int FN, int FM, int Q0, int Q1>
__device__ __forceinline__ void lowrank_mma(const GemmParams& p, v16f (&acc)[FN][FM], const LrFrags<FN, FM, Q1 - Q0>& f) {
#pragma unroll
  for (int q = Q0; q < Q1; ++q) {
    if (16 * q >= p.R) break;
    static_for<FN>([&](auto i) {
      static_for<FM>([&](auto j) {
        v8bf fa, fb;
        __builtin_memcpy(&fa, &f.wa[i][q - Q0], 16);
        __builtin_memcpy(&fb, &f.ub[j][q - Q0], 16);
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc[i][j], 0, 0, 0);
      });
    });
  }
}
// rank <= 64: every slice loaded, then the MFMAs
template <int FN, int FM>
__device__ __forceinline__ void lowrank_tile(const GemmParams& p, v16f (&acc)[FN][FM], int n_base, int m_base) {
  LrFrags<FN, FM, 4> f;
  lowrank_load<FN, FM, 0, 4>(p, f, n_base, m_base);
  lowrank_mma<FN, FM, 0, 4>(p, acc, f);
}

// ---------------------------------------------------------------------------------------------
// MX GEMM (W: E2M1, A: E2M1 or E4M3)
// ---------------------------------------------------------------------------------------------
template <int BM, int BN, bool AFP8>
struct MxTile {
  static_assert((BM == 128 || BM == 256) && (BN == 128 || BN == 256), "tile sizes");
  static constexpr int ACH = AFP8 ? 16 : 8;          // 16-byte chunks per A row per K chunk
  static constexpr int WROWB = 128, AROWB = ACH * 16;
  static constexpr int W_BYTES = BN * WROWB, A_BYTES = BM * AROWB;
  static constexpr int WS_BYTES = BN * 8, AS_BYTES = BM * 8;
  static constexpr int STAGE = W_BYTES + A_BYTES + WS_BYTES + AS_BYTES;
  static constexpr int FN = BN / 64, FM = BM / 64;    // 32x32 blocks per wave (2 x 2 waves)
  static constexpr int WLD = BN * 8 / 256, ALD = BM * ACH / 256;
};

// Register-staged kernel, K ordering inside a 256-element chunk: MFMA step s (0..3) takes the
// chunk's 32-element blocks s and 4 + s as its two scale blocks.  The scale of block b comes
// from the lanes of half b, so a lane of half h needs the E8M0 bytes of blocks 4h + s: the
// dword [4h, 4h+4) of the row's 8 chunk scales, op_sel s picking the byte.  FP4 lanes of half h
// hold their block whole; FP8 lanes split theirs (below).  LDS rows of 128 or 256 bytes.
template <int BM, int BN, bool AFP8, int S>
__device__ __forceinline__ void mx_step(const uint8_t* sW, const uint8_t* sA, int wn0, int wm0,
                                        const uint32_t (&wsc)[BN / 64],
                                        const uint32_t (&asc)[BM / 64],
                                        v16f (&acc)[BN / 64][BM / 64]) {
  using T = MxTile<BM, BN, AFP8>;
  const int lane = lane_id();
  const int r32 = lane & 31, h = lane >> 5;
  v8i wf[T::FN], af[T::FM];
#pragma unroll
  for (int i = 0; i < T::FN; ++i) {
    const int row = wn0 + 32 * i + r32;
    const uint4 d = *(const uint4*)(sW + swz(row, 4 * h + S, T::WROWB));
    wf[i] = v8i{(int)d.x, (int)d.y, (int)d.z, (int)d.w, 0, 0, 0, 0};
  }
#pragma unroll
  for (int j = 0; j < T::FM; ++j) {
    const int row = wm0 + 32 * j + r32;
    if (AFP8) {
      // An FP8 operand lane of half h carries, in bytes 0-15, elements 16h..16h+15 of the
      // MFMA's first 32-element block and, in bytes 16-31, the same elements of its second
      // block (an FP4 lane carries its own block whole).  With block 0 = K block S and block 1
      // = K block 4 + S of the chunk, that is 16-byte chunk 2S + h and chunk 8 + 2S + h.
      const uint4 d0 = *(const uint4*)(sA + swz(row, 2 * S + h, T::AROWB));
      const uint4 d1 = *(const uint4*)(sA + swz(row, 8 + 2 * S + h, T::AROWB));
      af[j] = v8i{(int)d0.x, (int)d0.y, (int)d0.z, (int)d0.w,
                  (int)d1.x, (int)d1.y, (int)d1.z, (int)d1.w};
    } else {
      const uint4 d = *(const uint4*)(sA + swz(row, 4 * h + S, T::AROWB));
      af[j] = v8i{(int)d.x, (int)d.y, (int)d.z, (int)d.w, 0, 0, 0, 0};
    }
  }
  static_for<T::FN>([&](auto i) {
    static_for<T::FM>([&](auto j) {
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          wf[i], af[j], acc[i][j], 4, AFP8 ? 0 : 4, S, (int)wsc[i], S, (int)asc[j]);
    });
  });
}

template <int BM, int BN, bool AFP8, bool KAL>
struct MxStage {
  using T = MxTile<BM, BN, AFP8>;
  uint4 w[T::WLD], a[T::ALD];
  uint2 ws, as;  // this thread's share of the chunk's scale bytes (8 or 4 bytes each)
};

template <int BM, int BN, bool AFP8, bool KAL>
__global__ void __launch_bounds__(256, 1) gemm_mx_kernel(GemmParams p) {
  using T = MxTile<BM, BN, AFP8>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * T::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wn0 = (wave >> 1) * (BN / 2), wm0 = (wave & 1) * (BM / 2);
  const int tiles_n = (p.N + BN - 1) / BN, tiles_m = (p.M + BM - 1) / BM;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int nkc = (p.K + KC - 1) / KC;
  const int kblocks = p.K >> 5;
  const uint32_t w_row = (uint32_t)p.K >> 1, a_row = AFP8 ? (uint32_t)p.K : ((uint32_t)p.K >> 1);
  const uint32_t s_row = (uint32_t)kblocks;

  auto clamp32 = [](uint64_t v) -> uint32_t { return v > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)v; };
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.w_codes + (int64_t)n0 * w_row, clamp32((uint64_t)(p.N - n0) * w_row));
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a_codes + (int64_t)m0 * a_row, clamp32((uint64_t)(p.M - m0) * a_row));
  const __amdgpu_buffer_rsrc_t rws = make_rsrc(p.w_scales + (int64_t)n0 * s_row, clamp32((uint64_t)(p.N - n0) * s_row));
  const __amdgpu_buffer_rsrc_t ras = make_rsrc(p.a_scales + (int64_t)m0 * s_row, clamp32((uint64_t)(p.M - m0) * s_row));

  // per-thread offsets of load i: row = i * (256 / CH) + tid / CH, chunk c = tid % CH
  const uint32_t voff_w = (uint32_t)(tid >> 3) * w_row + (uint32_t)(tid & 7) * 16u;
  const uint32_t voff_a = (uint32_t)(tid / T::ACH) * a_row + (uint32_t)(tid % T::ACH) * 16u;
  constexpr int W_ROWS_PER_LD = 256 / 8, A_ROWS_PER_LD = 256 / T::ACH;

  MxStage<BM, BN, AFP8, KAL> st;
  auto gload = [&](int kc) {
#pragma unroll
    for (int i = 0; i < T::WLD; ++i)
      st.w[i] = load16(rw, voff_w + (uint32_t)(i * W_ROWS_PER_LD) * w_row + (uint32_t)kc * 128u);
#pragma unroll
    for (int i = 0; i < T::ALD; ++i)
      st.a[i] = load16(ra, voff_a + (uint32_t)(i * A_ROWS_PER_LD) * a_row + (uint32_t)kc * T::AROWB);
    if (KAL) {
      // the tile's BN (BM) rows of 8 scale bytes are spread over all 256 threads
      if (BN == 256) st.ws = load8(rws, (uint32_t)tid * s_row + (uint32_t)kc * 8u);
      else st.ws = make_uint2(load4(rws, (uint32_t)(tid >> 1) * s_row + (uint32_t)kc * 8u + (tid & 1) * 4u), 0u);
      if (BM == 256) st.as = load8(ras, (uint32_t)tid * s_row + (uint32_t)kc * 8u);
      else st.as = make_uint2(load4(ras, (uint32_t)(tid >> 1) * s_row + (uint32_t)kc * 8u + (tid & 1) * 4u), 0u);
    } else {
      // K not a multiple of the chunk: the last chunk is partial.  Codes past the row end are
      // zeroed (reading them is in bounds: the next row, or past the buffer end, which reads 0)
      // and scale bytes are read one by one.
      const int kb0 = kc * 8;
#pragma unroll
      for (int i = 0; i < T::WLD; ++i)
        if (kb0 + (tid & 7) >= kblocks) st.w[i] = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < T::ALD; ++i)
        if (kb0 + (AFP8 ? (tid % T::ACH) >> 1 : tid % T::ACH) >= kblocks) st.a[i] = make_uint4(0, 0, 0, 0);
      uint32_t wlo = 0, whi = 0, alo = 0, ahi = 0;
      for (int b = 0; b < 8; ++b) {
        if (kb0 + b < kblocks) {
          const uint32_t vw = tid < BN ? load1(rws, (uint32_t)tid * s_row + (uint32_t)(kb0 + b)) : 0u;
          const uint32_t va = tid < BM ? load1(ras, (uint32_t)tid * s_row + (uint32_t)(kb0 + b)) : 0u;
          if (b < 4) { wlo |= vw << (8 * b); alo |= va << (8 * b); }
          else { whi |= vw << (8 * (b - 4)); ahi |= va << (8 * (b - 4)); }
        }
      }
      st.ws = make_uint2(wlo, whi);
      st.as = make_uint2(alo, ahi);
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* sW = smem + buf * T::STAGE;
    uint8_t* sA = sW + T::W_BYTES;
    uint8_t* sWS = sA + T::A_BYTES;
    uint8_t* sAS = sWS + T::WS_BYTES;
#pragma unroll
    for (int i = 0; i < T::WLD; ++i)
      *(uint4*)(sW + swz(i * W_ROWS_PER_LD + (tid >> 3), tid & 7, T::WROWB)) = st.w[i];
#pragma unroll
    for (int i = 0; i < T::ALD; ++i)
      *(uint4*)(sA + swz(i * A_ROWS_PER_LD + tid / T::ACH, tid % T::ACH, T::AROWB)) = st.a[i];
    if (KAL) {
      if (BN == 256) *(uint2*)(sWS + tid * 8) = st.ws;
      else *(uint32_t*)(sWS + tid * 4) = st.ws.x;
      if (BM == 256) *(uint2*)(sAS + tid * 8) = st.as;
      else *(uint32_t*)(sAS + tid * 4) = st.as.x;
    } else {
      if (tid < BN) *(uint2*)(sWS + tid * 8) = st.ws;
      if (tid < BM) *(uint2*)(sAS + tid * 8) = st.as;
    }
  };

  v16f acc[T::FN][T::FM];
  static_for<T::FN>([&](auto i) { static_for<T::FM>([&](auto j) { acc[i][j] = v16f{}; }); });

  gload(0);
  sstore(0);
  __syncthreads();
  const int r32 = lane & 31, h = lane >> 5;
  for (int kc = 0; kc < nkc; ++kc) {
    const int buf = kc & 1;
    // The loop body has no branch, so nothing can be sunk past the MFMAs: the chunk after the
    // last one is loaded and stored too (its buffer loads are bounds-checked, and that LDS
    // buffer is never read again).
    gload(kc + 1);
    __builtin_amdgcn_sched_barrier(0);  // issue the loads before this chunk's MFMAs
    {
      const uint8_t* sW = smem + buf * T::STAGE;
      const uint8_t* sA = sW + T::W_BYTES;
      const uint8_t* sWS = sA + T::A_BYTES;
      const uint8_t* sAS = sWS + T::WS_BYTES;
      uint32_t wsc[T::FN], asc[T::FM];
#pragma unroll
      for (int i = 0; i < T::FN; ++i) wsc[i] = *(const uint32_t*)(sWS + (wn0 + 32 * i + r32) * 8 + 4 * h);
#pragma unroll
      for (int j = 0; j < T::FM; ++j) asc[j] = *(const uint32_t*)(sAS + (wm0 + 32 * j + r32) * 8 + 4 * h);
      mx_step<BM, BN, AFP8, 0>(sW, sA, wn0, wm0, wsc, asc, acc);
      mx_step<BM, BN, AFP8, 1>(sW, sA, wn0, wm0, wsc, asc, acc);
      mx_step<BM, BN, AFP8, 2>(sW, sA, wn0, wm0, wsc, asc, acc);
      mx_step<BM, BN, AFP8, 3>(sW, sA, wn0, wm0, wsc, asc, acc);
    }
    // Keep the LDS stores of the next chunk (and their wait on its global loads) behind this
    // chunk's MFMAs: issuing the MFMAs takes as long as they run, so the loads issued above are
    // in flight for the whole MFMA block.
    __builtin_amdgcn_sched_barrier(0);
    sstore(buf ^ 1);
    __syncthreads();
  }

  static_for<T::FN>([&](auto i) {
    static_for<T::FM>([&](auto j) {
      const int nb = n0 + wn0 + 32 * i, mb = m0 + wm0 + 32 * j;
      v16f a = acc[i][j];
      if (p.R > 0) a = lowrank_block(p, a, nb, mb);
      if (nb < p.N && mb < p.M) epilogue_block(p, a, nb, mb);
    });
  });
}

// ---------------------------------------------------------------------------------------------
// MX GEMM, ring-staged (K a multiple of 128)
// ---------------------------------------------------------------------------------------------
// A BM x BN output tile per workgroup, its waves in 2 (m) x NWAVES/2 (n), each wave
// BM/2 x 32 FN, and an LDS ring of 128-element K chunks:
//  - two workgroups per compute unit (tiles up to 256 x 128 with 4 waves, or 256 x 256 with 8
//    waves in step) and a 3-deep ring: chunk kc + 2 is fetched by direct-to-LDS buffer loads
//    while chunk kc is multiplied, so two chunks of load latency are hidden, and the second
//    workgroup fills the MFMA pipe while one waits at its barrier or runs its epilogue;
//  - the ping-pong W4A4 tile (PP, 256 x 256, one workgroup of 8 waves per compute unit, a 4-deep
//    ring): waves 0-3 and 4-7 alternate between MFMA and memory phases (see the main loop).
//  Measured at 75600 x 5120 x 5120 against the 256 x 128 two-workgroup tile: 0.974 against
//  1.00 ms, with 1.74 against 2.70 GB of L2 fills (the larger tile moves fewer bytes per MFMA,
//  and the shader clock under the power limit rises from about 1.57 to 1.81 GHz).
//
// K ordering inside a 128-element chunk (four 32-element blocks): MFMA step s (0, 1) takes blocks
// s and 2 + s as its scale blocks 0 and 1.  An FP4 lane of half h holds block 2h + s whole (16
// bytes); an FP8 lane of half h holds elements 16h..16h+15 of both blocks.  The E8M0 bytes of a
// row's chunk are one dword (blocks 0..3); a lane of half h reads its bytes 2h, 2h + 1 and
// op_sel s picks block 2h + s.
//
// LDS rows (64 bytes for FP4 codes, 128 for FP8) hold 16-byte pieces XOR-swizzled by the row so
// that a quarter wave of 16-byte fragment reads (16 consecutive rows, one piece index) covers
// all 64 banks: piece ^ ((row >> 2) & 3) for 64-byte rows, piece ^ ((row >> 1) & 7) for 128-byte
// rows.  A load instruction fills 1 KB of consecutive LDS (16 or 8 rows), lane i slot i, so each
// lane fetches the global piece that the swizzle puts in its slot.
template <int BM, int BN, bool AFP8, bool WFP8 = false, bool PP = false>
struct RingTile {
  static_assert((BM == 128 || BM == 256) && (BN == 128 || BN == 256), "tile sizes");
  static_assert(!WFP8 || AFP8, "E4M3 weights are paired with E4M3 activations");
  static_assert(!PP || (BM == 256 && BN == 256 && !AFP8) || (BM == 128 && BN == 256 && AFP8 && WFP8),
                "ping-pong: 256 x 256 W4A4 or 128 x 256 W8A8 tiles");
#ifndef MX_RING_W256
#define MX_RING_W256 8
#endif
  // 2 (m) x NWAVES/2 (n) waves; a 256-wide tile has 8 waves of 128 x 64 or 4 of 128 x 128
  static constexpr int NWAVES = PP ? 8 : BN == 256 ? MX_RING_W256 : 4;
  static constexpr int KCR = 128;
  static constexpr int WROWB = WFP8 ? 128 : 64, AROWB = AFP8 ? 128 : 64;  // bytes per row and chunk
  static constexpr int W_BYTES = BN * WROWB, A_BYTES = BM * AROWB;
  static constexpr int WS_BYTES = BN * 4, AS_BYTES = BM * 4;
  static constexpr int STAGE = W_BYTES + A_BYTES + WS_BYTES + AS_BYTES;
  // ping-pong: 4 stages for W4A4; W8A8 stages are 49.5 KB, so 3 (chunk c + 2 loads in phase c)
  static constexpr int NSTAGE = PP && !WFP8 ? 4 : 3;
  static constexpr int LDS = NSTAGE * STAGE > BM * BN * 2 ? NSTAGE * STAGE : BM * BN * 2;
  static constexpr int WGS = 2 * LDS <= 160 * 1024 ? 2 : 1;  // workgroups per compute unit
  static constexpr int FN = BN / (NWAVES / 2) / 32, FM = BM / 64;  // 32x32 blocks per wave
  static constexpr int NW = W_BYTES / 1024 / NWAVES, NA = A_BYTES / 1024 / NWAVES;  // 1 KB loads
  static constexpr int TA = BM / 64, TW = BN / 64;                  // 256-byte scale loads
  static constexpr int NS = (TA + TW + NWAVES - 1) / NWAVES;        // scale loads per wave
  static constexpr int NDMA = NW + NA + NS;
  static_assert(LDS * WGS <= 160 * 1024, "LDS of the workgroups of a compute unit");
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// Workgroup barrier without the release fence of __syncthreads (which would wait for every load
// in flight, the prefetched chunks included); the memory clobber keeps LDS accesses on their side.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// Tile order for a grid of one tile per workgroup: XCD x = b % 8 gets a contiguous range of tile
// indices, walked in bands of GM tile rows (m), column by column.
template <int GM>
__device__ __forceinline__ void tile_coords_gm(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int q = total >> 3, r = total & 7;
  const int x = b & 7, j = b >> 3;
  const int t = x * q + min(x, r) + j;
  const int band = t / (GM * tiles_n);
  const int in = t - band * GM * tiles_n;
  const int rows = min(GM, tiles_m - band * GM);
  tm = band * GM + in % rows;
  tn = in / rows;
}

// BF16 output of a BM x BN ring-kernel tile through LDS (the ring is idle once the K loop is
// done): the tile is written as BM rows of 2 BN bytes, 16-byte chunks XOR-swizzled by the row,
// then stored as whole row segments (four 256-byte or two 512-byte rows per instruction)
// instead of 8-byte pieces of 32 rows.  Waves hold (BM/2) x 64 sub-tiles (2 x BN/64 waves).
template <int EPI, bool OUTF32>
__device__ __forceinline__ bool ring_staged_ok(const GemmParams& p) {
  return (EPI == EPI_BIAS || EPI == EPI_GELU) && !OUTF32 && (p.N % 8) == 0 && (p.ld_out % 8) == 0 &&
         (((uintptr_t)p.out) & 15) == 0;
}
template <int BM, int BN, int FN, int FM, int EPI, int NWAVES = BN / 32>
__device__ __forceinline__ void epilogue_ring_staged(const GemmParams& p, v16f (&acc)[FN][FM], uint8_t* smem,
                                                     int n0, int m0, int wn0, int wm0, int wave) {
  constexpr int RB = BN * 2, NCH = RB / 16;  // bytes and 16-byte chunks per staged row
  constexpr int RPI = 64 / NCH;              // rows per store instruction
  const int lane = lane_id();
  const int r32 = lane & 31, h = lane >> 5;
  static_for<FN>([&](auto i) {
    float b[16];
    load_bias16(p, n0 + wn0 + 32 * i, b);
    static_for<FM>([&](auto j) {
      __builtin_amdgcn_sched_barrier(0);
      float v[16];
      finish16<EPI>(p, acc[i][j], b, v);
      const int row = wm0 + 32 * j + r32;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = (wn0 + 32 * i) / 8 + g;  // 16-byte chunk of the row (8 BF16)
        const uint32_t lo = pack_bf16x2(v[4 * g], v[4 * g + 1]);
        const uint32_t hi = pack_bf16x2(v[4 * g + 2], v[4 * g + 3]);
        *(uint2*)(smem + row * RB + ((c ^ (row & (NCH - 1))) << 4) + 8 * h) = make_uint2(lo, hi);
      }
    });
  });
  wait_lds_all();
  barrier_only();
  const int c = lane % NCH;
  const int n = n0 + 8 * c;
#pragma unroll 4
  for (int it = 0; it < BM / NWAVES / RPI; ++it) {
    const int row = wave * (BM / NWAVES) + RPI * it + lane / NCH;
    const uint4 d = *(const uint4*)(smem + row * RB + ((c ^ (row & (NCH - 1))) << 4));
    const int m = m0 + row;
    // nontemporal: the output is not read again by this kernel (about 3 % faster than a
    // cached store at the 75600 x 5120 x 5120 shape)
    if (m < p.M && n < p.N)
      __builtin_nontemporal_store(u32x4{d.x, d.y, d.z, d.w}, (u32x4*)((uint16_t*)p.out + (int64_t)m * p.ld_out + n));
  }
}

template <int BM, int BN, bool AFP8, bool WFP8, int EPI, bool OUTF32, bool LR, bool PP = false>
__global__ void __launch_bounds__((RingTile<BM, BN, AFP8, WFP8, PP>::NWAVES * 64), (RingTile<BM, BN, AFP8, WFP8, PP>::WGS))
gemm_mx_ring_kernel(GemmParams p) {
  using T = RingTile<BM, BN, AFP8, WFP8, PP>;
  // Ping-pong: an operand constrained to an AGPR lets the register allocator place the MFMA
  // accumulators in AGPRs (about 1 % faster at 75600 x 5120 x 5120 than in VGPRs)
  if constexpr (PP) asm volatile("; accumulators in AGPRs" ::"a"(0.0f));
  typedef typename std::conditional<AFP8, v8i, v4i>::type AV;
  typedef typename std::conditional<WFP8, v8i, v4i>::type WV;
  __shared__ __attribute__((aligned(16))) uint8_t smem[T::LDS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r32 = lane & 31, h = lane >> 5;
  const int wn0 = (wave >> 1) * (32 * T::FN), wm0 = (wave & 1) * (BM / 2);
  const int tiles_n = (p.N + BN - 1) / BN, tiles_m = (p.M + BM - 1) / BM;
  int tm, tn;
  tile_coords_gm<PP ? MX_PP_GM : MX_RING_GM>(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int nkc = p.K / T::KCR;
  const uint32_t w_row = WFP8 ? (uint32_t)p.K : ((uint32_t)p.K >> 1), a_row = AFP8 ? (uint32_t)p.K : ((uint32_t)p.K >> 1);
  const uint32_t s_row = (uint32_t)p.K >> 5;

  // Operand addressing.  Every load is descriptor + per-lane VGPR offset (range-checked) + chunk
  // offset kc * step in the scalar offset.
  //  Row-major operands: the descriptor starts at the tile's first row and ends at the matrix
  //  end, so rows past M or N read as zero; the VGPR offset holds row * row_bytes + piece.
  //  Tiled operands: the tile's rows are all present (rows are padded to 256); each 1 KB (256 B)
  //  load is one contiguous tile of the layout, the VGPR offset is tile row * chunk count * 1 KB
  //  (256 B) + lane * 16 (4).
  auto clamp32 = [](uint64_t v) -> uint32_t { return v > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)v; };
  const uint64_t wn = (uint64_t)(p.N - n0), am = (uint64_t)(p.M - m0);
  const bool wt = p.w_tiled != 0, at = p.a_tiled != 0;
  constexpr int A_TROWS = AFP8 ? 8 : 16, W_TROWS = WFP8 ? 8 : 16;  // rows per 1 KB code tile
  const uint64_t kb1k = (uint64_t)nkc * 1024u, kb256 = (uint64_t)nkc * 256u;
  const v4i rw = wt ? make_rsrc_sgpr(p.w_codes + (int64_t)(n0 / W_TROWS) * kb1k, clamp32((uint64_t)(BN / W_TROWS) * kb1k))
                    : make_rsrc_sgpr(p.w_codes + (int64_t)n0 * w_row, clamp32(wn * w_row));
  const v4i ra = at ? make_rsrc_sgpr(p.a_codes + (int64_t)(m0 / A_TROWS) * kb1k, clamp32((uint64_t)(BM / A_TROWS) * kb1k))
                    : make_rsrc_sgpr(p.a_codes + (int64_t)m0 * a_row, clamp32(am * a_row));
  const v4i rws = wt ? make_rsrc_sgpr(p.w_scales + (int64_t)(n0 / 64) * kb256, clamp32((uint64_t)(BN / 64) * kb256))
                     : make_rsrc_sgpr(p.w_scales + (int64_t)n0 * s_row, clamp32(wn * s_row));
  const v4i ras = at ? make_rsrc_sgpr(p.a_scales + (int64_t)(m0 / 64) * kb256, clamp32((uint64_t)(BM / 64) * kb256))
                     : make_rsrc_sgpr(p.a_scales + (int64_t)m0 * s_row, clamp32(am * s_row));
  const uint32_t w_step = wt ? 1024u : (uint32_t)T::WROWB, a_step = at ? 1024u : (uint32_t)T::AROWB;
  const uint32_t ws_step = wt ? 256u : 4u, as_step = at ? 256u : 4u;

  // lane offsets of the row-major code loads: 64-byte rows, 16 per load; 128-byte rows, 8 per load
  const uint32_t pc64 = (uint32_t)((lane & 3) ^ ((lane >> 4) & 3)) * 16u;
  const uint32_t lt16 = (uint32_t)lane * 16u;
  auto off_code = [&](auto fp8, int tr, bool tiled, uint32_t row_bytes) -> uint32_t {
    if (tiled) return (uint32_t)tr * (uint32_t)kb1k + lt16;
    if constexpr (decltype(fp8)::value) {
      const int row = 8 * tr + (lane >> 3);
      return (uint32_t)row * row_bytes + (uint32_t)((lane & 7) ^ ((row >> 1) & 7)) * 16u;
    } else {
      return (uint32_t)(16 * tr + (lane >> 2)) * row_bytes + pc64;
    }
  };
  // load q of this wave covers W_TROWS (A_TROWS) rows of the tile
  auto off_w = [&](int q) { return off_code(std::integral_constant<bool, WFP8>{}, wave * T::NW + q, wt, w_row); };
  auto off_a = [&](int q) { return off_code(std::integral_constant<bool, AFP8>{}, wave * T::NA + q, at, a_row); };
  // scale load k of this wave: 64 rows of A scales (u < TA) or of W scales; surplus slots repeat
  // the last W load (the same bytes to the same place)
  auto scale_slot = [&](int k, int& urow, bool& is_a) {
    const int u = wave + T::NWAVES * k;
    is_a = u < T::TA;
    urow = is_a ? u : min(u - T::TA, T::TW - 1);
  };
  auto off_s = [&](int urow, bool tiled) {
    return tiled ? (uint32_t)urow * (uint32_t)kb256 + (uint32_t)lane * 4u : (uint32_t)(64 * urow + lane) * s_row;
  };

  const uint32_t lds0 = lds_addr_of(smem);
  auto issue_one = [&](auto qc, int kc, int st) {
    constexpr int Q = decltype(qc)::value;
    const bool live = kc < nkc;
    const uint32_t sW = lds0 + (uint32_t)(st * T::STAGE);
    const uint32_t sA = sW + T::W_BYTES, sWS = sA + T::A_BYTES, sAS = sWS + T::WS_BYTES;
    if constexpr (Q < T::NW) {
      v4i dw = rw; dw[2] = live ? dw[2] : 0;
      dma_lds16(dw, sW + (uint32_t)((wave * T::NW + Q) * 1024), off_w(Q), (uint32_t)kc * w_step);
    } else if constexpr (Q < T::NW + T::NA) {
      constexpr int q = Q - T::NW;
      v4i da = ra; da[2] = live ? da[2] : 0;
      dma_lds16(da, sA + (uint32_t)((wave * T::NA + q) * 1024), off_a(q), (uint32_t)kc * a_step);
    } else {
      constexpr int k = Q - T::NW - T::NA;
      int urow; bool is_a;
      scale_slot(k, urow, is_a);
      v4i dws = rws, das = ras; dws[2] = live ? dws[2] : 0; das[2] = live ? das[2] : 0;
      dma_lds4(is_a ? das : dws, (is_a ? sAS : sWS) + (uint32_t)(urow * 256), off_s(urow, is_a ? at : wt),
               (uint32_t)kc * (is_a ? as_step : ws_step));
    }
  };
  auto issue = [&](int kc, int st) { static_for<T::NDMA>([&](auto q) { issue_one(q, kc, st); }); };

  v16f acc[T::FN][T::FM];
  static_for<T::FN>([&](auto i) { static_for<T::FM>([&](auto j) { acc[i][j] = v16f{}; }); });
  // E4M3-activation tiles (W4A8, few K chunks per tile): the first 32 ranks of the low-rank
  // branch are loaded before the K loop, so their latency is hidden behind it
  constexpr bool LR_EARLY = LR && AFP8;
  LrFrags<T::FN, T::FM, 2> lr_early;
  if constexpr (LR_EARLY) lowrank_load<T::FN, T::FM, 0, 2>(p, lr_early, n0 + wn0, m0 + wm0);

  // fragment addresses inside a stage (step 0; step 1 is piece ^ 1)
  const int wrow = wn0 + r32, arow = wm0 + r32;  // + 32 i: the XOR term is unchanged

  // The fragments of a chunk (both MFMA steps) and its scale dwords, read from stage `stg`.
  struct Frags {
    uint32_t wsc[T::FN], asc[T::FM];
    WV wf[2][T::FN];
    AV af[2][T::FM];
  };
  // 16-byte pieces of a lane's fragment: E2M1 rows (64 bytes) hold the lane's 32-element block
  // whole in piece 2h + s; E4M3 rows (128 bytes) hold elements 16h..16h+15 of both blocks, in
  // pieces 2s + h and 4 + 2s + h.
  auto frag4 = [&](const uint8_t* base, int row, int s) -> v4i {
    return *(const v4i*)(base + row * 64 + (((2 * h + s) ^ ((row >> 2) & 3)) << 4));
  };
  auto frag8 = [&](const uint8_t* base, int row, int s) -> v8i {
    const int g = (row >> 1) & 7;
    const v4i d0 = *(const v4i*)(base + row * 128 + (((2 * s + h) ^ g) << 4));
    const v4i d1 = *(const v4i*)(base + row * 128 + (((4 + 2 * s + h) ^ g) << 4));
    return v8i{d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
  };
  auto read_chunk = [&](int stg, Frags& f) {
    const uint8_t* sW = smem + stg * T::STAGE;
    const uint8_t* sA = sW + T::W_BYTES;
    const uint8_t* sWS = sA + T::A_BYTES;
    const uint8_t* sAS = sWS + T::WS_BYTES;
    // the two E8M0 bytes of this lane's half (blocks 2h, 2h + 1 of the chunk): a 16-bit read at
    // byte 2h of the row's scale dword, op_sel picking the step's byte
#pragma unroll
    for (int i = 0; i < T::FN; ++i) f.wsc[i] = *(const uint16_t*)(sWS + (wrow + 32 * i) * 4 + 2 * h);
#pragma unroll
    for (int j = 0; j < T::FM; ++j) f.asc[j] = *(const uint16_t*)(sAS + (arow + 32 * j) * 4 + 2 * h);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int i = 0; i < T::FN; ++i) {
        if constexpr (WFP8) f.wf[s][i] = frag8(sW, wrow + 32 * i, s);
        else f.wf[s][i] = frag4(sW, wrow + 32 * i, s);
      }
#pragma unroll
      for (int j = 0; j < T::FM; ++j) {
        if constexpr (AFP8) f.af[s][j] = frag8(sA, arow + 32 * j, s);
        else f.af[s][j] = frag4(sA, arow + 32 * j, s);
      }
    }
  };
  // The MFMAs of step S, with the loads of chunk `dkc` into stage `dst` that fall in this step:
  // load q goes after MFMA (q + 1) * TOTAL / NDMA - 1 of the chunk's TOTAL (spread out; a burst
  // of loads would fill the vector-memory queue and hold up the MFMA issue behind it).  With
  // more loads than MFMAs the first slot takes two.
  constexpr int TOTAL = 2 * T::FN * T::FM;
  static_assert(2 * TOTAL >= T::NDMA, "two load slots per MFMA at most");
  constexpr auto dma_slot = [](int q) {
    const int m = (q + 1) * TOTAL / T::NDMA - 1;
    return m < 0 ? 0 : m;
  };
  auto mma_step = [&](auto sc, const Frags& f, int dkc, int dst) {
    constexpr int S = decltype(sc)::value;
    static_for<T::FN>([&](auto i) {
      static_for<T::FM>([&](auto j) {
        if constexpr (WFP8)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.wf[S][i], f.af[S][j], acc[i][j], 0, 0, S,
                                                                      (int)f.wsc[i], S, (int)f.asc[j]);
        else if constexpr (AFP8)
          acc[i][j] = mfma_scale_32x32x64_f4f8(f.wf[S][i], f.af[S][j], acc[i][j], 4, 0, S, (int)f.wsc[i], S, (int)f.asc[j]);
        else
          acc[i][j] = mfma_scale_32x32x64_f4f4(f.wf[S][i], f.af[S][j], acc[i][j], 4, 4, S, (int)f.wsc[i], S, (int)f.asc[j]);
        constexpr int M = S * T::FN * T::FM + decltype(i)::value * T::FM + decltype(j)::value;
        static_for<T::NDMA>([&](auto qc) {
          if constexpr (dma_slot(decltype(qc)::value) == M) {
            __builtin_amdgcn_sched_barrier(0);
            issue_one(qc, dkc, dst);
            __builtin_amdgcn_sched_barrier(0);
          }
        });
      });
    });
  };
  // loads issued during step 0 (those of a chunk that precede its step-1 MFMAs)
  constexpr int LOADS_S0 = [&] {
    int n = 0;
    for (int q = 0; q < T::NDMA; ++q) n += dma_slot(q) < TOTAL / 2 ? 1 : 0;
    return n;
  }();
  static_assert([&] {
    for (int q = 0; q < T::NDMA; ++q)
      if (dma_slot(q) >= TOTAL) return false;
    return true;
  }(), "every load has an MFMA slot");

  if constexpr (PP) {
    // Ping-pong: waves 0-3 (group 0) and 4-7 (group 1) put one wave of each group on every SIMD.
    // The groups alternate between an MFMA phase (the 16 MFMAs of one chunk on fragments already
    // in registers) and a memory phase (this wave's share of chunk c + 3's direct-to-LDS loads,
    // then the fragment reads of chunk c), with a workgroup barrier between phases, so the matrix
    // core of each SIMD is fed by one wave while the other waits on LDS and memory.
    //   phase 2c:     group 0 memory(c),     group 1 MFMA(c - 1)
    //   phase 2c + 1: group 0 MFMA(c),       group 1 memory(c)
    // Chunk c + D (D = stages - 1: 3 for W4A4, 2 for W8A8) goes into the stage of chunk c - 1,
    // whose last reads were in phases 2c - 2 and 2c - 1.  A memory phase ends by waiting for this
    // wave's loads of chunk c + 1 (the later ones may fly); the barrier after it publishes them
    // before chunk c + 1 is read (phase 2c + 2 at the earliest).
    static_assert(T::NSTAGE == 3 || T::NSTAGE == 4, "ping-pong ring depth");
    constexpr int D = T::NSTAGE - 1;  // a memory phase issues chunk c + D
    const bool g0 = wave < T::NWAVES / 2;
    static_for<D>([&](auto q) { issue(decltype(q)::value, decltype(q)::value); });
    wait_vmcnt<(D - 1) * T::NDMA>();  // chunk 0 landed
    barrier_only();
    Frags f;
    auto memory = [&](int c) {
      issue(c + D, (c + D) % T::NSTAGE);  // past the last chunk: empty loads (zero-range descriptors)
      read_chunk(c % T::NSTAGE, f);
      wait_vmcnt<(D - 1) * T::NDMA>();  // chunk c + 1 landed
      wait_lds_all();
    };
    auto mfma = [&]() {
      static_for<2>([&](auto sc) {
        constexpr int S = decltype(sc)::value;
        static_for<T::FN>([&](auto i) {
          static_for<T::FM>([&](auto j) {
            if constexpr (WFP8)
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.wf[S][i], f.af[S][j], acc[i][j], 0, 0, S,
                                                                          (int)f.wsc[i], S, (int)f.asc[j]);
            else
              acc[i][j] = mfma_scale_32x32x64_f4f4(f.wf[S][i], f.af[S][j], acc[i][j], 4, 4, S, (int)f.wsc[i], S,
                                                   (int)f.asc[j]);
          });
        });
      });
    };
    // One loop per group (the group is uniform per wave): each wave passes 2 nkc + 1 barriers.
    if (g0) {
      for (int c = 0; c < nkc; ++c) {
        memory(c);
        barrier_only();
        __builtin_amdgcn_sched_barrier(0);
        mfma();
        __builtin_amdgcn_sched_barrier(0);
        barrier_only();
      }
      barrier_only();  // phase 2 nkc: group 1's last MFMA phase
    } else {
      barrier_only();  // phase 0: group 0 reads chunk 0
      for (int c = 0; c < nkc; ++c) {
        memory(c);
        barrier_only();
        __builtin_amdgcn_sched_barrier(0);
        mfma();
        __builtin_amdgcn_sched_barrier(0);
        barrier_only();
      }
    }
  } else {
  // Software pipeline over chunks.  Iteration kc: step-0 MFMAs of chunk kc (its fragments were
  // read last iteration) while chunk kc + 2 starts loading into the stage of chunk kc - 1; then
  // the barrier that publishes chunk kc + 1 -- its wait overlaps the MFMAs already in the pipe --
  // and the reads of chunk kc + 1 under the step-1 MFMAs of chunk kc.  A stage is refilled only
  // after the barrier that follows every wave's last read of it (each wave drains its LDS reads
  // before each barrier).
  issue(0, 0);
  issue(1, 1);
  wait_vmcnt<T::NDMA>();
  barrier_only();
  Frags cur;
  read_chunk(0, cur);
  int st = 0;  // stage of chunk kc
  for (int kc = 0; kc < nkc; ++kc) {
    const int st1 = st == 2 ? 0 : st + 1;  // chunk kc + 1
    const int st2 = st == 0 ? 2 : st - 1;  // chunk kc + 2 (the stage of chunk kc - 1)
    __builtin_amdgcn_sched_barrier(0);
    mma_step(std::integral_constant<int, 0>{}, cur, kc + 2, st2);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<LOADS_S0>();  // chunk kc + 1 landed (only chunk kc + 2's first loads may fly)
    wait_lds_all();          // this wave's reads of chunk kc are done
    barrier_only();
    Frags nxt;
    read_chunk(st1, nxt);    // past the last chunk this reads a stale stage: unused
    __builtin_amdgcn_sched_barrier(0);
    mma_step(std::integral_constant<int, 1>{}, cur, kc + 2, st2);
    __builtin_amdgcn_sched_barrier(0);
    cur = nxt;
    st = st1;
  }
  }

  if constexpr (LR && LR_EARLY) {  // slices 0-1 (rank 32) were loaded before the loop
    lowrank_mma<T::FN, T::FM, 0, 2>(p, acc, lr_early);
    if (p.R > 32) {
      LrFrags<T::FN, T::FM, 2> f;
      lowrank_load<T::FN, T::FM, 2, 4>(p, f, n0 + wn0, m0 + wm0);
      lowrank_mma<T::FN, T::FM, 2, 4>(p, acc, f);
    }
  } else if constexpr (LR) {
    lowrank_tile<T::FN, T::FM>(p, acc, n0 + wn0, m0 + wm0);
  }
  if (ring_staged_ok<EPI, OUTF32>(p)) {
    static_assert(BM * BN * 2 <= T::LDS, "output tile fits the ring");
    wait_vmem_all();  // the (empty) loads issued for the chunks past the end have landed
    barrier_only();   // every wave is done with the ring
    epilogue_ring_staged<BM, BN, T::FN, T::FM, EPI, T::NWAVES>(p, acc, smem, n0, m0, wn0, wm0, wave);
  } else {
    epilogue_direct<T::FN, T::FM, EPI, OUTF32>(p, acc, n0 + wn0, m0 + wm0);
  }
}

// ---------------------------------------------------------------------------------------------
// NVFP4 GEMM: E2M1 codes with per-16 E4M3 scales, exact dequant to BF16, BF16 MFMA
// ---------------------------------------------------------------------------------------------
template <int BM, int BN>
struct NvTile {
  static constexpr int ROWB = 128;                   // 256 FP4 codes per row per K chunk
  static constexpr int W_BYTES = BN * ROWB, A_BYTES = BM * ROWB;
  static constexpr int WS_BYTES = BN * 16, AS_BYTES = BM * 16;  // 16 E4M3 scales per row
  static constexpr int STAGE = W_BYTES + A_BYTES + WS_BYTES + AS_BYTES;
  static constexpr int FN = BN / 64, FM = BM / 64;
  static constexpr int WLD = BN * 8 / 256, ALD = BM * 8 / 256;
};

// 8 E2M1 codes (one dword) times an E4M3 block scale, as 8 exact BF16 values
__device__ __forceinline__ v8bf nv_dequant8(uint32_t codes, float sb) {
  uint32_t out[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = e2m1_value((codes >> (8 * i)) & 0xFu) * sb;
    const float hi = e2m1_value((codes >> (8 * i + 4)) & 0xFu) * sb;
    out[i] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
  }
  v8bf r;
  __builtin_memcpy(&r, out, 16);
  return r;
}

template <int BM, int BN>
__global__ void __launch_bounds__(256, 1) gemm_nv_kernel(GemmParams p) {
  using T = NvTile<BM, BN>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * T::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wn0 = (wave >> 1) * (BN / 2), wm0 = (wave & 1) * (BM / 2);
  const int tiles_n = (p.N + BN - 1) / BN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int nkc = (p.K + KC - 1) / KC;
  const int kgroups = p.K >> 4;
  const int64_t row_b = p.K >> 1, s_row = kgroups;

  uint4 wreg[T::WLD], areg[T::ALD];
  uint4 wsreg = make_uint4(0, 0, 0, 0), asreg = make_uint4(0, 0, 0, 0);

  auto load_sc = [&](const uint8_t* src, int kc) -> uint4 {
    uint32_t w[4] = {0, 0, 0, 0};
    for (int b = 0; b < 16; ++b) {
      const uint32_t v = (kc * 16 + b < kgroups) ? src[b] : 0u;
      w[b >> 2] |= v << (8 * (b & 3));
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  };
  auto gload = [&](int kc) {
#pragma unroll
    for (int i = 0; i < T::WLD; ++i) {
      const int q = i * 256 + tid, row = q >> 3, c = q & 7;
      const int n = min(n0 + row, p.N - 1);
      const int kg = kc * 16 + 2 * c;  // a 16-byte chunk holds two 16-element groups
      wreg[i] = kg < kgroups
                    ? *(const uint4*)(p.w_codes + (int64_t)n * row_b + (int64_t)kc * 128 + c * 16)
                    : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < T::ALD; ++i) {
      const int q = i * 256 + tid, row = q >> 3, c = q & 7;
      const int m = min(m0 + row, p.M - 1);
      const int kg = kc * 16 + 2 * c;
      areg[i] = kg < kgroups
                    ? *(const uint4*)(p.a_codes + (int64_t)m * row_b + (int64_t)kc * 128 + c * 16)
                    : make_uint4(0, 0, 0, 0);
    }
    if (tid < BN) wsreg = load_sc(p.w_scales + (int64_t)min(n0 + tid, p.N - 1) * s_row + kc * 16, kc);
    if (tid < BM) asreg = load_sc(p.a_scales + (int64_t)min(m0 + tid, p.M - 1) * s_row + kc * 16, kc);
  };
  auto sstore = [&](int buf) {
    uint8_t* sW = smem + buf * T::STAGE;
    uint8_t* sA = sW + T::W_BYTES;
    uint8_t* sWS = sA + T::A_BYTES;
    uint8_t* sAS = sWS + T::WS_BYTES;
#pragma unroll
    for (int i = 0; i < T::WLD; ++i) {
      const int q = i * 256 + tid, row = q >> 3, c = q & 7;
      *(uint4*)(sW + swz(row, c, T::ROWB)) = wreg[i];
    }
#pragma unroll
    for (int i = 0; i < T::ALD; ++i) {
      const int q = i * 256 + tid, row = q >> 3, c = q & 7;
      *(uint4*)(sA + swz(row, c, T::ROWB)) = areg[i];
    }
    if (tid < BN) *(uint4*)(sWS + tid * 16) = wsreg;
    if (tid < BM) *(uint4*)(sAS + tid * 16) = asreg;
  };

  v16f acc[T::FN][T::FM];
#pragma unroll
  for (int i = 0; i < T::FN; ++i)
#pragma unroll
    for (int j = 0; j < T::FM; ++j) acc[i][j] = v16f{};

  gload(0);
  sstore(0);
  __syncthreads();
  const int r32 = lane & 31, h = lane >> 5;
  for (int kc = 0; kc < nkc; ++kc) {
    const int buf = kc & 1;
    if (kc + 1 < nkc) gload(kc + 1);
    const uint8_t* sW = smem + buf * T::STAGE;
    const uint8_t* sA = sW + T::W_BYTES;
    const uint8_t* sWS = sA + T::A_BYTES;
    const uint8_t* sAS = sWS + T::WS_BYTES;
    // group g covers K [16g, 16g+16) of the chunk: 8 bytes at row offset 8g; lane half h takes
    // elements 8h..8h+7, i.e. the dword at byte 8g + 4h (inside 16-byte chunk g/2).
    for (int g = 0; g < 16; ++g) {
      v8bf wf[T::FN], af[T::FM];
#pragma unroll
      for (int i = 0; i < T::FN; ++i) {
        const int row = wn0 + 32 * i + r32;
        const uint32_t c = *(const uint32_t*)(sW + swz(row, g >> 1, T::ROWB) + 8 * (g & 1) + 4 * h);
        wf[i] = nv_dequant8(c, e4m3_value(sWS[row * 16 + g]));
      }
#pragma unroll
      for (int j = 0; j < T::FM; ++j) {
        const int row = wm0 + 32 * j + r32;
        const uint32_t c = *(const uint32_t*)(sA + swz(row, g >> 1, T::ROWB) + 8 * (g & 1) + 4 * h);
        af[j] = nv_dequant8(c, e4m3_value(sAS[row * 16 + g]));
      }
      static_for<T::FN>([&](auto i) {
        static_for<T::FM>([&](auto j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i], af[j], acc[i][j], 0, 0, 0);
        });
      });
    }
    if (kc + 1 < nkc) sstore(buf ^ 1);
    __syncthreads();
  }

  static_for<T::FN>([&](auto i) {
    static_for<T::FM>([&](auto j) {
      const int nb = n0 + wn0 + 32 * i, mb = m0 + wm0 + 32 * j;
      if (nb < p.N && mb < p.M) epilogue_block(p, acc[i][j], nb, mb);
    });
  });
}

// ---------------------------------------------------------------------------------------------
// NVFP4 GEMM, ring-staged (K a multiple of 64)
// ---------------------------------------------------------------------------------------------
// The E4M3 per-16 block scales cannot ride in the scaled MFMA (E8M0 per 32 only), and code x
// block scale needs up to 6 significant bits.  Both are exact in FP16 (11 bits; magnitudes
// 2^-10 .. 2688), so each lane dequantizes its own fragments in registers with the gfx950
// conversions (two E2M1 codes -> two FP16, exact; two E4M3 scales -> two FP16, exact) and one
// packed FP16 multiply, and the product runs on V_MFMA_F32_32X32X16_F16.  The two FP32 global
// scales multiply the accumulator in the epilogue.
// Tile and waves as the MX ring kernel (256 x 128, 2 x 2 waves of 128 x 64, two workgroups per
// compute unit); K chunks of 64 (32 code bytes and 4 scale bytes per row) in a 4-deep LDS ring.
// K order inside a chunk: lane half h holds chunk elements 32h..32h+31 (16 contiguous bytes);
// MFMA step t (0..3) takes elements 32h + 8t .. 32h + 8t + 7, which lie in scale block 2h + t/2.
// LDS code rows are 32 bytes, the two 16-byte halves swapped on rows with bit 3 set, so that a
// quarter wave (16 consecutive rows, one half each) reads 16 distinct bank groups.
template <int BM, int BN>
struct NvRingTile {
  static_assert(BM == 256 && (BN == 128 || BN == 256), "tile sizes");
  static constexpr int WGS = 256 / BN;  // workgroups per compute unit (4 waves each)
  static constexpr int KCN = 64, ROWB = 32;
  static constexpr int W_BYTES = BN * ROWB, A_BYTES = BM * ROWB;
  static constexpr int WS_BYTES = BN * 4, AS_BYTES = BM * 4;
  static constexpr int STAGE = W_BYTES + A_BYTES + WS_BYTES + AS_BYTES;
  static constexpr int NSTAGE = 4;
  static constexpr int LDS = NSTAGE * STAGE > BM * BN * 2 ? NSTAGE * STAGE : BM * BN * 2;
  static constexpr int FN = BN / 64, FM = BM / 64;                 // 2 x 2 waves
  static constexpr int NW = W_BYTES / 4096, NA = A_BYTES / 4096;  // 1 KB loads per wave
  static constexpr int TA = BM / 64, TW = BN / 64;                 // 256-byte scale loads
  static constexpr int NS = (TA + TW + 3) / 4;
  static constexpr int NDMA = NW + NA + NS;
  static_assert(LDS * WGS <= 160 * 1024, "LDS of the workgroups of a compute unit");
};

// 8 E2M1 codes (one dword, element 2j in the low nibble of byte j) times a block scale, as 8
// exact FP16 values.  The conversion's scale operand only contributes its exponent, so it is 1
// and the block scale is a packed FP16 multiply (exact: at most 6 significant bits).
__device__ __forceinline__ v8h nv_dequant8_f16(uint32_t codes, v2h sb) {
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * sb;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * sb;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * sb;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * sb;
  return v8h{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

template <int BM, int BN, int EPI, bool OUTF32>
__global__ void __launch_bounds__(256, 256 / BN) gemm_nv_ring_kernel(GemmParams p) {
  using T = NvRingTile<BM, BN>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[T::LDS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r32 = lane & 31, h = lane >> 5;
  const int wn0 = (wave >> 1) * (BN / 2), wm0 = (wave & 1) * (BM / 2);
  const int tiles_n = (p.N + BN - 1) / BN, tiles_m = (p.M + BM - 1) / BM;
  int tm, tn;
  tile_coords_gm<MX_RING_GM>(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int nkc = p.K / T::KCN;
  const uint32_t row_b = (uint32_t)p.K >> 1, s_row = (uint32_t)p.K >> 4;

  // descriptors from the tile's first row to the matrix end (rows past M or N read as zero)
  auto clamp32 = [](uint64_t v) -> uint32_t { return v > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)v; };
  const uint64_t wn = (uint64_t)(p.N - n0), am = (uint64_t)(p.M - m0);
  const v4i rw = make_rsrc_sgpr(p.w_codes + (int64_t)n0 * row_b, clamp32(wn * row_b));
  const v4i ra = make_rsrc_sgpr(p.a_codes + (int64_t)m0 * row_b, clamp32(am * row_b));
  const v4i rws = make_rsrc_sgpr(p.w_scales + (int64_t)n0 * s_row, clamp32(wn * s_row));
  const v4i ras = make_rsrc_sgpr(p.a_scales + (int64_t)m0 * s_row, clamp32(am * s_row));
  // code loads: 32 rows of 32 bytes per 1 KB load, lane i -> row i/2, LDS half i&1
  const uint32_t half_lane = (uint32_t)((lane & 1) ^ ((lane >> 4) & 1)) * 16u;
  auto off_c = [&](int grp) { return (uint32_t)(32 * grp + (lane >> 1)) * row_b + half_lane; };
  auto scale_slot = [&](int k, int& urow, bool& is_a) {
    const int u = wave + 4 * k;
    is_a = u < T::TA;
    urow = is_a ? u : min(u - T::TA, T::TW - 1);
  };
  const uint32_t lds0 = lds_addr_of(smem);
  auto issue_one = [&](auto qc, int kc, int st) {
    constexpr int Q = decltype(qc)::value;
    const bool live = kc < nkc;
    const uint32_t sW = lds0 + (uint32_t)(st * T::STAGE);
    const uint32_t sA = sW + T::W_BYTES, sWS = sA + T::A_BYTES, sAS = sWS + T::WS_BYTES;
    if constexpr (Q < T::NW) {
      v4i d = rw;
      d[2] = live ? d[2] : 0;
      dma_lds16(d, sW + (uint32_t)((wave * T::NW + Q) * 1024), off_c(wave * T::NW + Q), (uint32_t)kc * 32u);
    } else if constexpr (Q < T::NW + T::NA) {
      constexpr int q = Q - T::NW;
      v4i d = ra;
      d[2] = live ? d[2] : 0;
      dma_lds16(d, sA + (uint32_t)((wave * T::NA + q) * 1024), off_c(wave * T::NA + q), (uint32_t)kc * 32u);
    } else {
      constexpr int k = Q - T::NW - T::NA;
      int urow;
      bool is_a;
      scale_slot(k, urow, is_a);
      v4i d = is_a ? ras : rws;
      d[2] = live ? d[2] : 0;
      dma_lds4(d, (is_a ? sAS : sWS) + (uint32_t)(urow * 256), (uint32_t)(64 * urow + lane) * s_row,
               (uint32_t)kc * 4u);
    }
  };

  v16f acc[T::FN][T::FM];
  static_for<T::FN>([&](auto i) { static_for<T::FM>([&](auto j) { acc[i][j] = v16f{}; }); });
  const int wrow = wn0 + r32, arow = wm0 + r32;  // + 32 i: the half swap (bit 3) is unchanged
  const uint32_t cpos_w = (uint32_t)(wrow * 32 + ((h ^ ((wrow >> 3) & 1)) << 4));
  const uint32_t cpos_a = (uint32_t)(arow * 32 + ((h ^ ((arow >> 3) & 1)) << 4));
  const uint32_t shift = 16u * (uint32_t)h;

  static_for<T::NSTAGE - 1>([&](auto i) {
    static_for<T::NDMA>([&](auto q) { issue_one(q, (int)decltype(i)::value, (int)decltype(i)::value); });
  });
  // The codes and scale pairs of a chunk, read from LDS stage `stg`.
  struct NvFrags {
    v4i wc[T::FN], ac[T::FM];
    v2h ws2[T::FN], as2[T::FM];  // the lane's two E4M3 block scales (elements 0-7, 8-15) as FP16
  };
  auto read_chunk = [&](int stg, NvFrags& f) {
    const uint8_t* sW = smem + stg * T::STAGE;
    const uint8_t* sA = sW + T::W_BYTES;
    const uint8_t* sWS = sA + T::A_BYTES;
    const uint8_t* sAS = sWS + T::WS_BYTES;
#pragma unroll
    for (int i = 0; i < T::FN; ++i) {
      f.wc[i] = *(const v4i*)(sW + cpos_w + i * 32 * 32);
      const uint32_t sb = *(const uint32_t*)(sWS + (wrow + 32 * i) * 4) >> shift;
      f.ws2[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb, 1.0f, false);
    }
#pragma unroll
    for (int j = 0; j < T::FM; ++j) {
      f.ac[j] = *(const v4i*)(sA + cpos_a + j * 32 * 32);
      const uint32_t sb = *(const uint32_t*)(sAS + (arow + 32 * j) * 4) >> shift;
      f.as2[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb, 1.0f, false);
    }
  };
  // Dequantized fragments, double-buffered over the four 16-element steps of a chunk: step
  // t + 1's fragments are dequantized between step t's MFMAs (one fragment after every
  // FN * FM / (FN + FM) MFMAs), so the conversions run while the matrix core is busy.
  v8h wf[2][T::FN], af[2][T::FM];
  auto dequant_frag = [&](const NvFrags& f, auto tq, auto kq, auto bq) {
    constexpr int t = decltype(tq)::value, k = decltype(kq)::value, b = decltype(bq)::value;
    // steps 0-1 (elements 0-7 of the lane's 16) take the first block scale, steps 2-3 the second
    if constexpr (k < T::FN) {
      const v2h sc = t < 2 ? __builtin_shufflevector(f.ws2[k], f.ws2[k], 0, 0) : __builtin_shufflevector(f.ws2[k], f.ws2[k], 1, 1);
      wf[b][k] = nv_dequant8_f16((uint32_t)f.wc[k][t], sc);
    } else {
      const v2h sc = t < 2 ? __builtin_shufflevector(f.as2[k - T::FN], f.as2[k - T::FN], 0, 0)
                           : __builtin_shufflevector(f.as2[k - T::FN], f.as2[k - T::FN], 1, 1);
      af[b][k - T::FN] = nv_dequant8_f16((uint32_t)f.ac[k - T::FN][t], sc);
    }
  };
  constexpr int TOTAL = 4 * T::FN * T::FM;
  // The MFMAs of step t of a chunk, with the dequantization of the next step (step 0 of the next
  // chunk, from fn, after step 3) and the loads of chunk `dkc` into stage `dst` that fall in this
  // step (load q after MFMA (q + 1) * TOTAL / NDMA - 1).
  auto mma_step = [&](auto tc, const NvFrags& f, const NvFrags& fn, int dkc, int dst) {
    constexpr int t = decltype(tc)::value;
    constexpr int cb = t & 1;
    static_for<T::FN>([&](auto i) {
      static_for<T::FM>([&](auto j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[cb][i], af[cb][j], acc[i][j], 0, 0, 0);
        constexpr int Mi = decltype(i)::value * T::FM + decltype(j)::value;  // MFMA index in the step
        constexpr int M = t * T::FN * T::FM + Mi;
        constexpr int PER = T::FN * T::FM / (T::FN + T::FM);  // MFMAs per dequantized fragment
        if constexpr ((Mi + 1) % PER == 0 && (Mi + 1) / PER <= T::FN + T::FM) {
          __builtin_amdgcn_sched_barrier(0);
          dequant_frag(t < 3 ? f : fn, std::integral_constant<int, (t + 1) & 3>{},
                       std::integral_constant<int, (Mi + 1) / PER - 1>{}, std::integral_constant<int, cb ^ 1>{});
          __builtin_amdgcn_sched_barrier(0);
        }
        static_for<T::NDMA>([&](auto qc) {
          if constexpr ((decltype(qc)::value + 1) * TOTAL / T::NDMA - 1 == M) {
            __builtin_amdgcn_sched_barrier(0);
            issue_one(qc, dkc, dst);
            __builtin_amdgcn_sched_barrier(0);
          }
        });
      });
    });
  };
  // loads of a chunk issued during steps 0 and 1
  constexpr int LOADS_H0 = [] {
    int n = 0;
    for (int q = 0; q < T::NDMA; ++q) n += (q + 1) * TOTAL / T::NDMA - 1 < TOTAL / 2 ? 1 : 0;
    return n;
  }();

  // Software pipeline over chunks.  Iteration kc: steps 0-1 of chunk kc (its codes were read
  // last iteration) while chunk kc + 3 starts loading into the stage of chunk kc - 1; then the
  // barrier that publishes chunk kc + 1 (its wait overlaps the MFMAs in flight) and the reads of
  // chunk kc + 1 under steps 2-3 of chunk kc.  A stage is refilled only after the barrier that
  // follows every wave's last read of it.
  NvFrags cur;
  wait_vmcnt<(T::NSTAGE - 2) * T::NDMA>();  // chunk 0 landed
  barrier_only();
  read_chunk(0, cur);
  static_for<T::FN + T::FM>([&](auto kq) {  // step 0 of chunk 0 (later chunks: under step 3)
    dequant_frag(cur, std::integral_constant<int, 0>{}, kq, std::integral_constant<int, 0>{});
  });
  int st = 0;  // stage of chunk kc
  for (int kc = 0; kc < nkc; ++kc) {
    const int stn = st == 0 ? T::NSTAGE - 1 : st - 1;  // the stage of chunk kc - 1: chunk kc + 3
    const int st1 = st == T::NSTAGE - 1 ? 0 : st + 1;  // chunk kc + 1
    __builtin_amdgcn_sched_barrier(0);
    mma_step(std::integral_constant<int, 0>{}, cur, cur, kc + T::NSTAGE - 1, stn);
    mma_step(std::integral_constant<int, 1>{}, cur, cur, kc + T::NSTAGE - 1, stn);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<(T::NSTAGE - 3) * T::NDMA + LOADS_H0>();  // chunk kc + 1 landed
    wait_lds_all();  // this wave's reads of chunk kc are done
    barrier_only();
    NvFrags nxt;
    read_chunk(st1, nxt);  // past the last chunk this reads a stage never written: unused
    __builtin_amdgcn_sched_barrier(0);
    mma_step(std::integral_constant<int, 2>{}, cur, nxt, kc + T::NSTAGE - 1, stn);
    mma_step(std::integral_constant<int, 3>{}, cur, nxt, kc + T::NSTAGE - 1, stn);
    __builtin_amdgcn_sched_barrier(0);
    cur = nxt;
    st = st1;
  }

  if (ring_staged_ok<EPI, OUTF32>(p)) {
    wait_vmem_all();
    barrier_only();
    epilogue_ring_staged<BM, BN, T::FN, T::FM, EPI, 4>(p, acc, smem, n0, m0, wn0, wm0, wave);
  } else {
    epilogue_direct<T::FN, T::FM, EPI, OUTF32>(p, acc, n0 + wn0, m0 + wm0);
  }
}

// ---------------------------------------------------------------------------------------------
// low-rank down projection u = bf16(x . down_t^T): one workgroup of 4 waves per 32 (m) x 32 (r)
// block, wave w summing its own contiguous quarter of K.  A wave streams its 32 rows of x and of
// down_t through a private 4-stage LDS ring of 64-element K chunks with direct-to-LDS loads: one
// 1 KB load is 8 rows x 128 bytes, so every cache line is fetched whole by one instruction, and
// three chunks (24 KB per wave) stay in flight.  One 32x32x16 BF16 MFMA
// per 16 elements; the four partial sums are added in the fixed order w = 0..3 (deterministic).
// LDS rows of 128 bytes hold their 16-byte pieces XOR-swizzled by ((row >> 1) & 7).
// ---------------------------------------------------------------------------------------------
constexpr int LR_WAVES = 4, LR_STG = 4, LR_KC = 64;
constexpr int LR_HALF = 32 * LR_KC * 2;  // 32 rows x 128 bytes: one operand of a stage
constexpr int LR_STAGE = 2 * LR_HALF;

// QUANT: the same pass also quantizes x to MXFP8 in the tiled layout (codes, scales; rows of the
// 32-row blocks, the tiled padding beyond them is not written), from the x chunks already in LDS,
// so the W4A8 linear reads its activation once for both the quantizer and the low-rank branch.
template <bool QUANT>
__global__ void __launch_bounds__(LR_WAVES * 64) lowrank_down_kernel(const uint16_t* __restrict__ x,
                                                                     int64_t ld_x,
                                                                     const uint16_t* __restrict__ down_t,
                                                                     int M, int K, int R,
                                                                     uint16_t* __restrict__ u,
                                                                     uint8_t* __restrict__ codes,
                                                                     uint8_t* __restrict__ scales) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[LR_WAVES * LR_STG * LR_STAGE];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, r32 = lane & 31;
  const int rb = blockIdx.y * 32, mb = blockIdx.x * 32;
  auto clamp32 = [](uint64_t v) -> uint32_t { return v > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)v; };
  // descriptors end at the last element of the block's last row: rows past M (R) and the
  // elements past K of that row read as zero
  const int xrows = min(32, M - mb), drows = min(32, R - rb);
  const uint64_t xrow = (uint64_t)ld_x * 2, drow = (uint64_t)K * 2;
  const v4i rx = make_rsrc_sgpr(x + (int64_t)mb * ld_x, clamp32((uint64_t)(xrows - 1) * xrow + drow));
  const v4i rd = make_rsrc_sgpr(down_t + (int64_t)rb * K, clamp32((uint64_t)drows * drow));

  const int nchunks = (K + LR_KC - 1) / LR_KC;
  const int per = (nchunks + LR_WAVES - 1) / LR_WAVES;
  const int cbeg = min(nchunks, wave * per), nc = min(nchunks, cbeg + per) - cbeg;

  // load i of a chunk: rows 8i + lane / 8, LDS slot lane % 8 <- global piece slot ^ swizzle
  uint32_t vx[4], vd[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 8 * i + (lane >> 3);
    const uint32_t piece = (uint32_t)((lane & 7) ^ ((row >> 1) & 7));
    vx[i] = (uint32_t)row * (uint32_t)xrow + piece * 16u;
    vd[i] = (uint32_t)row * (uint32_t)drow + piece * 16u;
  }
  const uint32_t lds_w = lds_addr_of(smem) + (uint32_t)(wave * LR_STG * LR_STAGE);
  auto issue = [&](int c, int stg) {
    v4i ax = rx, ad = rd;
    if (c >= nc) { ax[2] = 0; ad[2] = 0; }  // past this wave's range: zero-filling empty loads
    const uint32_t soff = (uint32_t)((cbeg + c) * LR_KC * 2);
    const uint32_t sx = lds_w + (uint32_t)(stg * LR_STAGE);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma_lds16(ax, sx + (uint32_t)(i * 1024), vx[i], soff);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma_lds16(ad, sx + (uint32_t)(LR_HALF + i * 1024), vd[i], soff);
  };

  v16f acc = v16f{};
  issue(0, 0);
  issue(1, 1);
  issue(2, 2);
  const int swz = (r32 >> 1) & 7;
  for (int c = 0; c < nc; ++c) {
    wait_vmcnt<16>();  // chunk c landed; chunks c + 1 and c + 2 (8 loads each) may still fly
    asm volatile("" ::: "memory");
    const uint8_t* sx = smem + (wave * LR_STG + (c & 3)) * LR_STAGE;
    const uint8_t* sd = sx + LR_HALF;
    const int k0 = (cbeg + c) * LR_KC;
    v4i fx[4], fd[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int off = r32 * 128 + (((2 * j + h) ^ swz) << 4);
      fx[j] = *(const v4i*)(sx + off);
      fd[j] = *(const v4i*)(sd + off);
      if (k0 + 16 * j + 8 * h >= K) {  // past K (K % 32 == 0, so only whole pieces)
        fx[j] = v4i{0, 0, 0, 0};
        fd[j] = v4i{0, 0, 0, 0};
      }
    }
    if constexpr (QUANT) {
      if (blockIdx.y == 0) {  // one rank block quantizes (uniform)
        // this lane's group: row r32, elements 32h .. 32h + 31 of the chunk = pieces 4h .. 4h + 3
        uint32_t w[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const v4i d = *(const v4i*)(sx + r32 * 128 + (((4 * h + q) ^ swz) << 4));
          w[4 * q] = (uint32_t)d[0];
          w[4 * q + 1] = (uint32_t)d[1];
          w[4 * q + 2] = (uint32_t)d[2];
          w[4 * q + 3] = (uint32_t)d[3];
        }
        uint32_t cw[8], sbyte;
        quant_fp8_group32(w, cw, sbyte);
        const int kg = k0 + 32 * h;  // first element of the group
        if (kg < K) {
          const int64_t r = mb + r32, kb = kg >> 7, nkc = K >> 7;
          const int g16 = (kg & 127) >> 4;  // first 16-element piece of the group in its tile
          *(uint4*)(codes + tiled_fp8_off(r, kb, g16, nkc)) = make_uint4(cw[0], cw[1], cw[2], cw[3]);
          *(uint4*)(codes + tiled_fp8_off(r, kb, g16 + 1, nkc)) = make_uint4(cw[4], cw[5], cw[6], cw[7]);
          scales[tiled_scale_off(r, kb, nkc) + ((kg & 127) >> 5)] = (uint8_t)sbyte;
        }
      }
    }
    issue(c + 3, (c + 3) & 3);  // into the stage of chunk c - 1, read last iteration
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v8bf fa, fb;
      __builtin_memcpy(&fa, &fd[j], 16);
      __builtin_memcpy(&fb, &fx[j], 16);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc, 0, 0, 0);
    }
  }
  wait_vmem_all();
  __syncthreads();  // every wave's loads and reads of the ring are done
  float* part = (float*)smem;  // [LR_WAVES - 1][16][64]
  if (wave > 0) {
#pragma unroll
    for (int e = 0; e < 16; ++e) part[((wave - 1) * 16 + e) * 64 + lane] = acc[e];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < LR_WAVES - 1; ++w)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] += part[(w * 16 + e) * 64 + lane];
  const int mo = mb + r32;
  if (mo >= M) return;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int ro = rb + 8 * (e >> 2) + 4 * h + (e & 3);
    if (ro < R) u[(int64_t)mo * R + ro] = (uint16_t)f32_to_bf16_rne(acc[e]);
  }
}

// ---------------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------------
// PP: the ping-pong schedule of the 256 x 256 W4A4 tile (MX_RING_PP=0 turns it off) and of the
// 128 x 256 W8A8 tile (MX_W8_PP).
#ifndef MX_RING_PP
#define MX_RING_PP 1
#endif
#ifndef MX_W8_PP
#define MX_W8_PP 0
#endif
template <int BM, int BN, bool AFP8, bool WFP8, int EPI, bool OUTF32, bool LR>
static void run_ring(const GemmParams& p, int grid, hipStream_t s) {
  constexpr bool PP = (MX_RING_PP && BM == 256 && BN == 256 && !AFP8 && !WFP8 && !LR) ||
                      (MX_W8_PP && BM == 128 && BN == 256 && AFP8 && WFP8 && !LR);
  gemm_mx_ring_kernel<BM, BN, AFP8, WFP8, EPI, OUTF32, LR, PP>
      <<<grid, RingTile<BM, BN, AFP8, WFP8, PP>::NWAVES * 64, 0, s>>>(p);
}

// Every (epilogue, output type, low-rank) combination of the ring kernel.
template <int BM, int BN, bool AFP8, bool WFP8, int EPI, bool LR>
static void run_ring_o(const GemmParams& p, int grid, hipStream_t s) {
  if constexpr (EPI == EPI_GELU_QUANT || EPI == EPI_GELU_QUANT_T) run_ring<BM, BN, AFP8, WFP8, EPI, false, LR>(p, grid, s);
  else if (p.out_f32) run_ring<BM, BN, AFP8, WFP8, EPI, true, LR>(p, grid, s);
  else run_ring<BM, BN, AFP8, WFP8, EPI, false, LR>(p, grid, s);
}
template <int BM, int BN, bool AFP8, bool WFP8, bool LR>
static void run_ring_e(const GemmParams& p, int grid, hipStream_t s) {
  if constexpr (!AFP8) {  // the tiled re-quantized output needs the 256-row tiles of W4A4
    if (p.epi == EPI_GELU_QUANT_T) {
      run_ring_o<BM, BN, AFP8, WFP8, EPI_GELU_QUANT_T, LR>(p, grid, s);
      return;
    }
  }
  if (p.epi == EPI_GELU_QUANT) run_ring_o<BM, BN, AFP8, WFP8, EPI_GELU_QUANT, LR>(p, grid, s);
  else if (p.epi == EPI_GELU) run_ring_o<BM, BN, AFP8, WFP8, EPI_GELU, LR>(p, grid, s);
  else run_ring_o<BM, BN, AFP8, WFP8, EPI_BIAS, LR>(p, grid, s);
}

// K % 128 == 0: the ring kernel (row-major or tiled operands); otherwise the register-staged
// kernel, which reads row-major operands (the tiled layout implies K % 128 == 0).
// The ping-pong tile needs one 256 x 256 tile per compute unit of the MI355X (256) to pay: with
// fewer tiles the 256 x 128 two-workgroup tile spreads the work over more compute units.
constexpr int PP_MIN_TILES = 256;

template <int BM, int BN, bool AFP8>
static hipError_t run_mx(const GemmParams& p, hipStream_t s) {
  if (p.K % 128 == 0) {
#ifndef MX_RING_BN
#define MX_RING_BN 128
#endif
    // W4A4 without a low-rank branch on a large grid: the 256 x 256 ping-pong tile (one workgroup
    // of 8 waves per compute unit); otherwise 256 x MX_RING_BN (W4A4) or 128 x 128 (W4A8), two
    // workgroups per compute unit
    if constexpr (!AFP8 && MX_RING_PP) {
      const int tiles_pp = ((p.M + 255) / 256) * ((p.N + 255) / 256);
      if (p.R == 0 && tiles_pp >= PP_MIN_TILES) {
        run_ring_e<256, 256, false, false, false>(p, tiles_pp, s);
        return hipGetLastError();
      }
    }
    constexpr int RBN = AFP8 ? 128 : MX_RING_BN;
    const int tiles = ((p.M + BM - 1) / BM) * ((p.N + RBN - 1) / RBN);
    if (p.R > 0) run_ring_e<BM, RBN, AFP8, false, true>(p, tiles, s);
    else run_ring_e<BM, RBN, AFP8, false, false>(p, tiles, s);
  } else {
    const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    gemm_mx_kernel<BM, BN, AFP8, false><<<tiles, 256, 0, s>>>(p);
  }
  return hipGetLastError();
}

// MXFP8 x MXFP8 (W8A8): the ring kernel only; the caller checks K % 128 == 0.  A 128 x 256 tile
// with 8 waves (one workgroup per compute unit, 148.5 KB of LDS): 12 % faster than 256 x 128
// and 30 % faster than 128 x 128 at 75600 x 5120 x 5120.
#ifndef MX_W8_BM
#define MX_W8_BM 128
#endif
#ifndef MX_W8_BN
#define MX_W8_BN 256
#endif
static hipError_t run_w8a8(const GemmParams& p, hipStream_t s) {
  constexpr int BM = MX_W8_BM, BN = MX_W8_BN;
  const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  if (p.R > 0) run_ring_e<BM, BN, true, true, true>(p, tiles, s);
  else run_ring_e<BM, BN, true, true, false>(p, tiles, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Small W4A4 linears in one launch: quantize A and multiply
// ---------------------------------------------------------------------------------------------
// When the grid of the ring kernels would be a handful of tiles, the two launches (quantizer,
// GEMM) and their load latencies are most of the time.  A workgroup of 4 waves takes a 64 x 64
// output tile: it loads its 64 weight rows (codes and scales) and quantizes its 64 activation
// rows, each lane one 32-element group with the standalone quantizer's rule, into LDS; then each
// wave multiplies one 32 x 32 block over the whole K and runs the common epilogue.  The MFMA of
// chunk c, step s pairs blocks 4c + s (lanes 0-31) and 4c + 2 + s (lanes 32-63), in the ring
// kernels' order, with one accumulator chained through K from zero, so the output bits equal
// those of the quantizer + ring GEMM pair.  K % 128 == 0, K <= FS_KMAX (the LDS holds the tile's
// codes for the whole K, within the 64 KB of dynamic LDS a launch gets by default); A rows past M
// and W rows past N read as zero.
constexpr int FS_KMAX = 896;
constexpr int FS_IT = 64 * (FS_KMAX / 32) / 256;  // 32-element blocks per thread at K = FS_KMAX
constexpr int FS_MAX_TILES = 8;  // ring tiles (256 x 128) up to which the one-launch path is taken

bool linear_fused_small_ok(const GemmParams& p) {
  const int64_t ring_tiles = (int64_t)((p.M + 255) / 256) * ((p.N + 127) / 128);
  return p.R == 0 && (p.epi == EPI_BIAS || p.epi == EPI_GELU) && p.K % 128 == 0 && p.K <= FS_KMAX &&
         p.M > 0 && ring_tiles <= FS_MAX_TILES;
}

__global__ void __launch_bounds__(256) linear_fused_small_kernel(GemmParams p, const uint16_t* __restrict__ a,
                                                                 int64_t ld_a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t fs_lds[];
  const int K = p.K, kbs = K / 32;      // 32-element blocks per row
  const int pitch = K / 2 + 16;         // code bytes per LDS row (+16: rows fall in different banks)
  uint8_t* sW = fs_lds;                 // [64][pitch] weight codes
  uint8_t* sA = sW + 64 * pitch;        // [64][pitch] activation codes
  uint8_t* sWs = sA + 64 * pitch;       // [64][kbs] weight scale bytes
  uint8_t* sAs = sWs + 64 * kbs;        // [64][kbs] activation scale bytes
  const int tiles_n = (p.N + 63) / 64;
  const int m0 = (blockIdx.x / tiles_n) * 64, n0 = (blockIdx.x % tiles_n) * 64;
  const int64_t nkc = K >> 7;
  // Thread t takes blocks i = t + 256 j (row i / kbs, 32-element block i % kbs), j < nit: 64 kbs
  // is a multiple of 256 (K % 128 == 0), so every thread has exactly nit of them.  All their
  // loads are issued first (rows past M or N read the last valid row and are zeroed after), so
  // the workgroup waits for memory once rather than once per block.
  const int nit = 64 * kbs / 256;  // <= FS_IT
  uint4 wcv[FS_IT], av[FS_IT][4];
  uint32_t wsv[FS_IT];
#pragma unroll
  for (int j = 0; j < FS_IT; ++j) {
    if (j >= nit) break;  // uniform
    const int i = threadIdx.x + 256 * j, r = i / kbs, kb = i - r * kbs;
    const int n = min(n0 + r, p.N - 1), m = min(m0 + r, p.M - 1);
    if (p.w_tiled) {
      wcv[j] = *(const uint4*)(p.w_codes + tiled_fp4_off(n, kb >> 2, kb & 3, nkc));
      wsv[j] = p.w_scales[tiled_scale_off(n, kb >> 2, nkc) + (kb & 3)];
    } else {
      wcv[j] = *(const uint4*)(p.w_codes + (int64_t)n * (K / 2) + kb * 16);
      wsv[j] = p.w_scales[(int64_t)n * kbs + kb];
    }
    const uint16_t* src = a + (int64_t)m * ld_a + kb * 32;
#pragma unroll
    for (int q = 0; q < 4; ++q) av[j][q] = *(const uint4*)(src + 8 * q);
  }
#pragma unroll
  for (int j = 0; j < FS_IT; ++j) {
    if (j >= nit) break;
    const int i = threadIdx.x + 256 * j, r = i / kbs, kb = i - r * kbs;
    // weight block: 16 code bytes and one scale byte (row-major or tiled operand layout)
    const bool nin = n0 + r < p.N, min_ = m0 + r < p.M;
    *(uint4*)(sW + r * pitch + kb * 16) = nin ? wcv[j] : make_uint4(0u, 0u, 0u, 0u);
    sWs[r * kbs + kb] = (uint8_t)(nin ? wsv[j] : 0u);
    // activation group: 32 BF16 values, quantized in this lane
    uint32_t w[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      w[4 * q] = min_ ? av[j][q].x : 0u;
      w[4 * q + 1] = min_ ? av[j][q].y : 0u;
      w[4 * q + 2] = min_ ? av[j][q].z : 0u;
      w[4 * q + 3] = min_ ? av[j][q].w : 0u;
    }
    uint32_t ac[4], asb;
    quant_fp4_group32(w, ac, asb);
    *(uint4*)(sA + r * pitch + kb * 16) = make_uint4(ac[0], ac[1], ac[2], ac[3]);
    sAs[r * kbs + kb] = (uint8_t)asb;
  }
  __syncthreads();
  const int lane = lane_id(), r32 = lane & 31, h = lane >> 5;
  const int wave = threadIdx.x >> 6;
  const int wn = 32 * (wave & 1), wm = 32 * (wave >> 1);
  const uint8_t* wrow = sW + (wn + r32) * pitch;
  const uint8_t* arow = sA + (wm + r32) * pitch;
  const uint8_t* wsrow = sWs + (wn + r32) * kbs;
  const uint8_t* asrow = sAs + (wm + r32) * kbs;
  v16f acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
  for (int c = 0; c < K / 128; ++c) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int kb = 4 * c + 2 * h + st;
      const v4i wf = *(const v4i*)(wrow + kb * 16);
      const v4i af = *(const v4i*)(arow + kb * 16);
      acc = mfma_scale_32x32x64_f4f4(wf, af, acc, 4, 4, 0, (int)wsrow[kb], 0, (int)asrow[kb]);
    }
  }
  epilogue_block(p, acc, n0 + wn, m0 + wm);
}

hipError_t launch_linear_fused_small(const GemmParams& p, const uint16_t* a, int64_t ld_a, hipStream_t s) {
  if (!linear_fused_small_ok(p)) return hipErrorInvalidValue;
  const int tiles = ((p.M + 63) / 64) * ((p.N + 63) / 64);
  const size_t lds = (size_t)2 * 64 * (p.K / 2 + 16) + (size_t)2 * 64 * (p.K / 32);
  hipLaunchKernelGGL(linear_fused_small_kernel, dim3(tiles), dim3(256), lds, s, p, a, ld_a);
  return hipGetLastError();
}

hipError_t launch_gemm_mx(const GemmParams& p, bool act_fp8, bool w_fp8, hipStream_t s) {
  if (p.M == 0) return hipSuccess;
  if (w_fp8) return p.K % 128 == 0 && act_fp8 ? run_w8a8(p, s) : hipErrorInvalidValue;
  if (act_fp8) return run_mx<128, 256, true>(p, s);
  return run_mx<256, 256, false>(p, s);
}

#ifndef NV_RING_BN
#define NV_RING_BN 256
#endif
template <int EPI>
static void run_nv_ring(const GemmParams& p, int grid, hipStream_t s) {
  constexpr int BN = NV_RING_BN;
  if constexpr (EPI == EPI_GELU_QUANT) gemm_nv_ring_kernel<256, BN, EPI, false><<<grid, 256, 0, s>>>(p);
  else if (p.out_f32) gemm_nv_ring_kernel<256, BN, EPI, true><<<grid, 256, 0, s>>>(p);
  else gemm_nv_ring_kernel<256, BN, EPI, false><<<grid, 256, 0, s>>>(p);
}

// K % 64 == 0: the ring kernel; otherwise the register-staged kernel (K a multiple of 16).
hipError_t launch_gemm_nv(const GemmParams& p, hipStream_t s) {
  if (p.M == 0) return hipSuccess;
  if (p.K % 64 == 0) {
    const int tiles = ((p.M + 255) / 256) * ((p.N + NV_RING_BN - 1) / NV_RING_BN);
    if (p.epi == EPI_GELU_QUANT) run_nv_ring<EPI_GELU_QUANT>(p, tiles, s);
    else if (p.epi == EPI_GELU) run_nv_ring<EPI_GELU>(p, tiles, s);
    else run_nv_ring<EPI_BIAS>(p, tiles, s);
  } else {
    const int tiles = ((p.M + 255) / 256) * ((p.N + 255) / 256);
    gemm_nv_kernel<256, 256><<<tiles, 256, 0, s>>>(p);
  }
  return hipGetLastError();
}

hipError_t launch_lowrank_down(const uint16_t* x, int64_t ld_x, const uint16_t* down_t, int M,
                               int K, int R, uint16_t* u, hipStream_t s) {
  if (M == 0) return hipSuccess;
  dim3 grid((M + 31) / 32, (R + 31) / 32);
  lowrank_down_kernel<false><<<grid, LR_WAVES * 64, 0, s>>>(x, ld_x, down_t, M, K, R, u, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_quant8_lowrank_down(const uint16_t* x, int64_t ld_x, const uint16_t* down_t, int M,
                                      int K, int R, uint16_t* u, uint8_t* codes, uint8_t* scales,
                                      hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (K % 128) return hipErrorInvalidValue;  // the tiled layout
  dim3 grid((M + 31) / 32, (R + 31) / 32);
  lowrank_down_kernel<true><<<grid, LR_WAVES * 64, 0, s>>>(x, ld_x, down_t, M, K, R, u, codes, scales);
  return hipGetLastError();
}

}  // namespace mxk
