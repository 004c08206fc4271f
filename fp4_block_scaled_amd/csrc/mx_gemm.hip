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
// K ordering inside a 256-element K chunk: the sum over k is order-free, so MFMA step s (0..3)
// takes the chunk's 32-element blocks s and 4 + s as its two scale blocks.  The scale of block
// b comes from the lanes of half b (lane / 32), so a lane of half h needs the E8M0 bytes of
// blocks 4h + s, s = 0..3: the contiguous dword [4h, 4h+4) of the row's 8 chunk scales, op_sel
// s picking the byte.  FP4 lanes of half h hold their block whole (64 contiguous bytes per row
// and chunk); FP8 lanes split theirs (see mx_step).  Both operands pair the same k.
//
// Staging: a 256 x 256 output tile per workgroup (4 waves, 128 x 128 each, 4 x 4 MFMA blocks),
// K chunks of 256 double-buffered in LDS.  LDS rows hold 16-byte chunks XOR-swizzled by the
// row index so that the 16-byte fragment reads of 8 consecutive rows hit distinct banks.
//
// NVFP4 (NVFP4 model card, Model Details) has E4M3 scales per 16 elements that the scaled MFMA
// cannot apply, and code * scale needs up to 6 significant bits, more than FP8 holds; it is
// dequantized exactly to BF16 after staging and run on V_MFMA_F32_32X32X16_BF16, with the
// product of the two FP32 global scales applied in the epilogue.
#include "mx_common.h"
#include "mx_internal.h"

#include <stdlib.h>

namespace mxk {

constexpr int KC = 256;  // K elements per staged chunk

__device__ __forceinline__ float gelu_tanh_f32(float y) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  return 0.5f * y * (1.0f + tanhf(c * (y + 0.044715f * y * y * y)));
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
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int n = nb + 8 * a + 4 * h;
    if (p.bias && n + 3 < p.N) {
      const uint2 u = *(const uint2*)(p.bias + n);
      b[4 * a + 0] = f16_to_f32(u.x & 0xFFFFu);
      b[4 * a + 1] = f16_to_f32(u.x >> 16);
      b[4 * a + 2] = f16_to_f32(u.y & 0xFFFFu);
      b[4 * a + 3] = f16_to_f32(u.y >> 16);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) b[4 * a + i] = (p.bias && n + i < p.N) ? f16_to_f32(p.bias[n + i]) : 0.0f;
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
      const uint32_t b0 = f32_to_bf16_rne(v[4 * a]), b1 = f32_to_bf16_rne(v[4 * a + 1]);
      const uint32_t b2 = f32_to_bf16_rne(v[4 * a + 2]), b3 = f32_to_bf16_rne(v[4 * a + 3]);
      if (n + 3 < p.N) {
        *(uint2*)o = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
      } else {
        const uint32_t bb[4] = {b0, b1, b2, b3};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (n + i < p.N) o[i] = (uint16_t)bb[i];
      }
    }
  }
}

// MXFP4 re-quantization of h along n: the 32 values of a block for row m live in lanes l and
// l ^ 32.  Same rule as the activation quantizer, on binary32 values.  Requires N % 32 == 0.
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
  const float inv = __uint_as_float((uint32_t)(127 - ex) << 23);
  uint32_t run[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    uint32_t r = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t u = __float_as_uint(v[4 * a + i]);
      const float q = __uint_as_float(u & 0x7FFFFFFFu) * inv;
      r |= (e2m1_code(q) | ((u >> 28) & 8u)) << (4 * i);
    }
    run[a] = bad ? 0u : r;  // 4 codes = 2 bytes at byte offset 4a + 2h of the block
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
  if (m < p.M && nb < p.N) {
    uint8_t* codes = (uint8_t*)p.out;
    *(uint2*)(codes + (int64_t)m * (p.N >> 1) + (nb >> 1) + 8 * h) = make_uint2(d0, d1);
    if (h == 0)
      p.out_scales[(int64_t)m * (p.N >> 5) + (nb >> 5)] = bad ? (uint8_t)0xFF : (uint8_t)(ex + 127);
  }
}

// One block through the compile-time epilogue.
template <int EPI, bool OUTF32>
__device__ __forceinline__ void epilogue_block_t(const GemmParams& p, const v16f& acc, const float (&b)[16],
                                                 int nb, int mb) {
  float v[16];
  finish16<EPI>(p, acc, b, v);
  if (EPI == EPI_GELU_QUANT) requant_block(p, v, nb, mb);
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

// Output of one wave's sub-tile through LDS, for the BF16 / FP32 epilogues when N, ld_out and out
// are 16-byte granular.  The 16 values a lane holds per 32 x 32 block are 4 runs of 4 consecutive
// n in one row, so direct stores put 16-byte pieces of 32 rows in each instruction.  Instead the
// values go to a (32 FM)-row x 128-byte LDS buffer (64 BF16 / 32 FP32 columns, 16-byte chunks
// XOR-swizzled by row), and each store instruction writes 8 whole 128-byte row segments.
// `stage` is this wave's (32 FM) x 128 bytes; only this wave touches it.
template <int FN, int FM, int EPI, bool OUTF32>
__device__ __forceinline__ void epilogue_staged(const GemmParams& p, v16f (&acc)[FN][FM], int n_base,
                                                int m_base, uint8_t* stage) {
  const int lane = lane_id();
  const int r32 = lane & 31, h = lane >> 5;
  auto sw = [](int row, int c) { return row * 128 + ((c ^ ((row ^ (row >> 3)) & 7)) << 4); };
  constexpr int PER_PASS = OUTF32 ? 1 : 2;  // n-blocks per 128-byte row segment
  static_for<FN / PER_PASS>([&](auto pass) {
    static_for<PER_PASS>([&](auto ii) {
      constexpr int I = decltype(pass)::value * PER_PASS + decltype(ii)::value;
      const int col0 = decltype(ii)::value * 32;
      float b[16];
      load_bias16(p, n_base + 32 * I, b);
      static_for<FM>([&](auto j) {
        __builtin_amdgcn_sched_barrier(0);  // one block at a time: keep register use small
        float v[16];
        finish16<EPI>(p, acc[I][j], b, v);
        const int row = 32 * j + r32;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int col = col0 + 8 * a + 4 * h;  // first of 4 consecutive columns
          if (OUTF32) {
            *(float4*)(stage + sw(row, col >> 2)) = make_float4(v[4 * a], v[4 * a + 1], v[4 * a + 2], v[4 * a + 3]);
          } else {
            const uint32_t b0 = f32_to_bf16_rne(v[4 * a]) | (f32_to_bf16_rne(v[4 * a + 1]) << 16);
            const uint32_t b1 = f32_to_bf16_rne(v[4 * a + 2]) | (f32_to_bf16_rne(v[4 * a + 3]) << 16);
            *(uint2*)(stage + sw(row, col >> 3) + ((col & 4) << 1)) = make_uint2(b0, b1);
          }
        }
      });
    });
    wait_lds_all();  // the wave's own LDS writes are done
    constexpr int ESZ = OUTF32 ? 4 : 2;
    const int ncol0 = n_base + decltype(pass)::value * (OUTF32 ? 32 : 64);
#pragma unroll
    for (int t = 0; t < FM * 4; ++t) {
      const int row = t * 8 + (lane >> 3), c = lane & 7;
      const uint4 d = *(const uint4*)(stage + sw(row, c));
      const int m = m_base + row;
      const int n = ncol0 + c * (16 / ESZ);
      if (m < p.M && n < p.N) *(uint4*)((uint8_t*)p.out + ((int64_t)m * p.ld_out + n) * ESZ) = d;
    }
    wait_lds_all();  // reads done before the next pass writes
  });
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
        if (mb < p.M) epilogue_block_t<EPI, OUTF32>(p, acc[i][j], b, nb, mb);
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

// Global -> register staging of one K chunk.  Buffer loads: the descriptor of each operand
// starts at the tile's first row and ends at the matrix end, so rows past M or N read as zero
// without clamping, and every load of a thread shares one VGPR offset pattern.
// Fragments of one MFMA step (see mx_step), split into an LDS load and the MFMAs so that the
// loads of step s+1 can be in flight while the MFMAs of step s issue.
template <int BM, int BN, bool AFP8>
struct MxFrags {
  typedef typename std::conditional<AFP8, v8i, v4i>::type AV;
  v4i w[BN / 64];
  AV a[BM / 64];
};

// One scaled MFMA: weight fragment (FP4) x activation fragment (FP4 or FP8).
template <bool AFP8, int S>
__device__ __forceinline__ v16f mx_mfma(const v4i& w, const typename MxFrags<256, 256, AFP8>::AV& a,
                                        const v16f& c, uint32_t ws, uint32_t as) {
  if constexpr (AFP8) return mfma_scale_32x32x64_f4f8(w, a, c, 4, 0, S, (int)ws, S, (int)as);
  else return mfma_scale_32x32x64_f4f4(w, a, c, 4, 4, S, (int)ws, S, (int)as);
}

template <int BM, int BN, bool AFP8, int S>
__device__ __forceinline__ void mx_load(const uint8_t* sW, const uint8_t* sA, int wn0, int wm0,
                                        MxFrags<BM, BN, AFP8>& f) {
  using T = MxTile<BM, BN, AFP8>;
  const int lane = lane_id();
  const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int i = 0; i < T::FN; ++i) {
    const int row = wn0 + 32 * i + r32;
    f.w[i] = *(const v4i*)(sW + swz(row, 4 * h + S, T::WROWB));
  }
#pragma unroll
  for (int j = 0; j < T::FM; ++j) {
    const int row = wm0 + 32 * j + r32;
    if constexpr (AFP8) {
      const v4i d0 = *(const v4i*)(sA + swz(row, 2 * S + h, T::AROWB));
      const v4i d1 = *(const v4i*)(sA + swz(row, 8 + 2 * S + h, T::AROWB));
      f.a[j] = v8i{d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
    } else {
      f.a[j] = *(const v4i*)(sA + swz(row, 4 * h + S, T::AROWB));
    }
  }
}

// The MFMAs of step S for weight row-block I only (FM instructions).
template <int BM, int BN, bool AFP8, int S, int I>
__device__ __forceinline__ void mx_mma_row(const MxFrags<BM, BN, AFP8>& f, const uint32_t (&wsc)[BN / 64],
                                           const uint32_t (&asc)[BM / 64],
                                           v16f (&acc)[BN / 64][BM / 64]) {
  using T = MxTile<BM, BN, AFP8>;
  static_for<T::FM>([&](auto j) { acc[I][j] = mx_mfma<AFP8, S>(f.w[I], f.a[j], acc[I][j], wsc[I], asc[j]); });
}

template <int BM, int BN, bool AFP8, int S>
__device__ __forceinline__ void mx_mma(const MxFrags<BM, BN, AFP8>& f, const uint32_t (&wsc)[BN / 64],
                                       const uint32_t (&asc)[BM / 64],
                                       v16f (&acc)[BN / 64][BM / 64]) {
  using T = MxTile<BM, BN, AFP8>;
  static_for<T::FN>([&](auto i) {
    static_for<T::FM>([&](auto j) { acc[i][j] = mx_mfma<AFP8, S>(f.w[i], f.a[j], acc[i][j], wsc[i], asc[j]); });
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

// Persistent schedule: workgroup b stays on XCD b % 8 and walks that XCD's contiguous range of
// tiles (see tile_coords) with a stride of the XCD's workgroup count.
struct XcdSchedule {
  int start, count, stride, first;
};
__device__ __forceinline__ XcdSchedule xcd_schedule(int total) {
  const int x = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int q = total >> 3, r = total & 7;
  XcdSchedule s;
  s.start = x * q + min(x, r);
  s.count = q + (x < r ? 1 : 0);
  s.stride = ((int)gridDim.x - x + 7) >> 3;  // workgroups on this XCD
  s.first = slot;
  return s;
}
__device__ __forceinline__ void band_coords(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GM = 4;
  const int band = t / (GM * tiles_n);
  const int in = t - band * GM * tiles_n;
  const int rows = min(GM, tiles_m - band * GM);
  tm = band * GM + in % rows;
  tn = in / rows;
}

// The MX GEMM with chunks staged by direct-to-LDS buffer loads (K a multiple of the chunk).  Each
// load instruction of a wave writes 64 consecutive 16-byte LDS slots, so a lane fetches the
// global chunk that belongs in its slot under the row swizzle: no VGPR staging, no LDS store
// instructions.  One workgroup per CU runs persistently over its tiles; the loads of the next
// chunk -- the next tile's first chunk at the end of a tile -- fly while the current chunk is
// multiplied, so a tile's start costs no load latency.
template <int BM, int BN, bool AFP8, int EPI, bool OUTF32, bool LR>
__global__ void __launch_bounds__(256, 1) gemm_mx_dma_kernel(GemmParams p) {
  using T = MxTile<BM, BN, AFP8>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * T::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn0 = (wave >> 1) * (BN / 2), wm0 = (wave & 1) * (BM / 2);
  const int tiles_n = (p.N + BN - 1) / BN, tiles_m = (p.M + BM - 1) / BM;
  const XcdSchedule sched = xcd_schedule(tiles_m * tiles_n);
  if (sched.first >= sched.count) return;
  const int nkc = p.K / KC;
  const uint32_t w_row = (uint32_t)p.K >> 1, a_row = AFP8 ? (uint32_t)p.K : ((uint32_t)p.K >> 1);
  const uint32_t s_row = (uint32_t)p.K >> 5;
  // staged output: 16-byte pieces of whole rows ((BM / 2) rows x 128 bytes per wave fit the free
  // chunk buffer)
  constexpr int ESZ = OUTF32 ? 4 : 2;
  const bool staged_out = EPI != EPI_GELU_QUANT && (p.N % (16 / ESZ)) == 0 &&
                          (p.ld_out % (16 / ESZ)) == 0 && (((uintptr_t)p.out) & 15) == 0;
  static_assert(4 * (BM / 2) * 128 <= T::STAGE, "staging area fits a chunk buffer");

  // buffer descriptors of one tile: they start at the tile's first row and end at the matrix
  // end, so rows past M or N read as zero; an absent tile gets empty descriptors
  struct TileDesc {
    v4i w, a, ws, as;
    int m0, n0;
  };
  auto clamp32 = [](uint64_t v) -> uint32_t { return v > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)v; };
  auto describe = [&](int j, bool present) {
    int tm, tn;
    band_coords(sched.start + j, tiles_m, tiles_n, tm, tn);
    TileDesc d;
    d.m0 = tm * BM;
    d.n0 = tn * BN;
    const uint64_t wn = present ? (uint64_t)(p.N - d.n0) : 0, am = present ? (uint64_t)(p.M - d.m0) : 0;
    d.w = make_rsrc_sgpr(p.w_codes + (int64_t)d.n0 * w_row, clamp32(wn * w_row));
    d.a = make_rsrc_sgpr(p.a_codes + (int64_t)d.m0 * a_row, clamp32(am * a_row));
    d.ws = make_rsrc_sgpr(p.w_scales + (int64_t)d.n0 * s_row, clamp32(wn * s_row));
    d.as = make_rsrc_sgpr(p.a_scales + (int64_t)d.m0 * s_row, clamp32(am * s_row));
    return d;
  };

  // Load instructions per wave and chunk: W codes BN/32 (1 KB each), A codes BM*ACH/256,
  // W / A scales BN/128, BM/128 (4-byte loads, 256 B each).  Lane offsets are recomputed at
  // each load (a few integer ops) rather than held in registers across the tile.
  constexpr int NW = BN / 32, NA = BM * T::ACH / 256, NWS = BN / 128, NAS = BM / 128;
  constexpr int A_RPI = 64 / T::ACH;  // A rows per load instruction
  auto off_w = [&](int i) {
    const int row = (wave * NW + i) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((row ^ (row >> 3)) & 7);
    return (uint32_t)row * w_row + (uint32_t)c * 16u;
  };
  auto off_a = [&](int i) {
    const int row = (wave * NA + i) * A_RPI + lane / T::ACH;
    const int c = (lane % T::ACH) ^ (T::ACH == 8 ? ((row ^ (row >> 3)) & 7) : (row & 15));
    return (uint32_t)row * a_row + (uint32_t)c * 16u;
  };
  auto off_s = [&](int base_row) { return (uint32_t)(base_row + (lane >> 1)) * s_row + (uint32_t)(lane & 1) * 4u; };

  const uint32_t lds0 = lds_addr_of(smem);
  // Load instruction q of a chunk (0 <= q < NDMA), in the order W codes, A codes, W scales,
  // A scales; issued in small groups between the MFMAs so that the vector-memory queue never
  // backs up into the MFMA issue.
  constexpr int NDMA = NW + NA + NWS + NAS;
  auto dma_one = [&](auto qc, const TileDesc& d, int kc, int buf) {
    constexpr int q = decltype(qc)::value;
    const uint32_t sW = lds0 + (uint32_t)(buf * T::STAGE);
    const uint32_t sA = sW + T::W_BYTES, sWS = sA + T::A_BYTES, sAS = sWS + T::WS_BYTES;
    if constexpr (q < NW) {
      dma_lds16(d.w, sW + (uint32_t)((wave * NW + q) * 1024), off_w(q), (uint32_t)kc * 128u);
    } else if constexpr (q < NW + NA) {
      constexpr int i = q - NW;
      dma_lds16(d.a, sA + (uint32_t)((wave * NA + i) * 1024), off_a(i), (uint32_t)(kc * T::AROWB));
    } else if constexpr (q < NW + NA + NWS) {
      constexpr int i = q - NW - NA;
      dma_lds4(d.ws, sWS + (uint32_t)((wave * NWS + i) * 256), off_s((wave * NWS + i) * 32), (uint32_t)kc * 8u);
    } else {
      constexpr int i = q - NW - NA - NWS;
      dma_lds4(d.as, sAS + (uint32_t)((wave * NAS + i) * 256), off_s((wave * NAS + i) * 32), (uint32_t)kc * 8u);
    }
  };
  auto dma = [&](const TileDesc& d, int kc, int buf) {
    static_for<NDMA>([&](auto q) { dma_one(q, d, kc, buf); });
  };
  // instructions [LO, HI) of the chunk
  auto dma_range = [&](auto lo, auto hi, const TileDesc& d, int kc, int buf) {
    static_for<decltype(hi)::value - decltype(lo)::value>([&](auto q) {
      dma_one(std::integral_constant<int, decltype(lo)::value + decltype(q)::value>{}, d, kc, buf);
    });
  };

  const int r32 = lane & 31, h = lane >> 5;
  auto load_scales = [&](int buf, uint32_t (&wsc)[T::FN], uint32_t (&asc)[T::FM]) {
    const uint8_t* sWS = smem + buf * T::STAGE + T::W_BYTES + T::A_BYTES;
    const uint8_t* sAS = sWS + T::WS_BYTES;
#pragma unroll
    for (int i = 0; i < T::FN; ++i) wsc[i] = *(const uint32_t*)(sWS + (wn0 + 32 * i + r32) * 8 + 4 * h);
#pragma unroll
    for (int j = 0; j < T::FM; ++j) asc[j] = *(const uint32_t*)(sAS + (wm0 + 32 * j + r32) * 8 + 4 * h);
  };
  auto sw_of = [&](int buf) { return (const uint8_t*)smem + buf * T::STAGE; };
  auto sa_of = [&](int buf) { return (const uint8_t*)smem + buf * T::STAGE + T::W_BYTES; };

  // Software pipeline: the LDS loads of MFMA step s+1 are issued before the MFMAs of step s, and
  // the barrier that publishes chunk kc+1 sits between the loads and the MFMAs of step 3 of
  // chunk kc, so the barrier and the first loads of kc+1 overlap those MFMAs.  The chunk loop
  // body is one basic block, so nothing moves across its scheduling barriers: each tile's first
  // pass multiplies zero fragments for the (absent) step 3 of chunk -1.
  v16f acc[T::FN][T::FM];
  MxFrags<BM, BN, AFP8> f0, f1;
  uint32_t wsc[T::FN], asc[T::FM], wsc3[T::FN], asc3[T::FM];

  int j = sched.first;
  TileDesc cur = describe(j, true);
  int gc = 0;  // chunks staged so far (LDS buffer parity)
  dma(cur, 0, 0);
  wait_vmem_all();
  __syncthreads();
  load_scales(0, wsc, asc);
  mx_load<BM, BN, AFP8, 0>(sw_of(0), sa_of(0), wn0, wm0, f0);
  while (true) {
    const int jn = j + sched.stride;
    const bool has_next = jn < sched.count;
    const TileDesc nxt = describe(has_next ? jn : j, has_next);
    static_for<T::FN>([&](auto i) { static_for<T::FM>([&](auto jj) { acc[i][jj] = v16f{}; }); });
#pragma unroll
    for (int i = 0; i < T::FN; ++i) { f1.w[i] = v4i{}; wsc3[i] = 0; }
#pragma unroll
    for (int jj = 0; jj < T::FM; ++jj) { f1.a[jj] = typename MxFrags<BM, BN, AFP8>::AV{}; asc3[jj] = 0; }
    // nothing of the compiler's own may be in flight inside the chunk loop: a wait it would
    // insert there for, say, a register reload would also wait for the chunk loads
    wait_vmem_all();
    for (int kc = 0; kc < nkc; ++kc, ++gc) {
      const int buf = gc & 1;
      // the next chunk: this tile's kc + 1, or the next tile's chunk 0 (empty descriptors past
      // the last tile).  Its buffer held chunk gc - 1, which every wave finished reading before
      // the last barrier.
      const bool last = kc + 1 == nkc;
      const TileDesc& dd = last ? nxt : cur;
      const int dkc = last ? 0 : kc + 1;
      // The loads of the next chunk are spread over the first three MFMA steps of this pass
      // (one group after each weight row-block), the fourth step covers their latency.
      constexpr int NPART = 3 * T::FN;
      auto mma_dma = [&](auto sc, auto part0, const MxFrags<BM, BN, AFP8>& f, const uint32_t (&ws_)[T::FN],
                         const uint32_t (&as_)[T::FM]) {
        static_for<T::FN>([&](auto i) {
          mx_mma_row<BM, BN, AFP8, decltype(sc)::value, decltype(i)::value>(f, ws_, as_, acc);
          __builtin_amdgcn_sched_barrier(0);
          constexpr int P = decltype(part0)::value + decltype(i)::value;
          dma_range(std::integral_constant<int, P * NDMA / NPART>{},
                    std::integral_constant<int, (P + 1) * NDMA / NPART>{}, dd, dkc, buf ^ 1);
          __builtin_amdgcn_sched_barrier(0);
        });
      };
      mma_dma(std::integral_constant<int, 3>{}, std::integral_constant<int, 0>{}, f1, wsc3, asc3);
      mx_load<BM, BN, AFP8, 1>(sw_of(buf), sa_of(buf), wn0, wm0, f1);
      __builtin_amdgcn_sched_barrier(0);
      mma_dma(std::integral_constant<int, 0>{}, std::integral_constant<int, T::FN>{}, f0, wsc, asc);
      mx_load<BM, BN, AFP8, 2>(sw_of(buf), sa_of(buf), wn0, wm0, f0);
      __builtin_amdgcn_sched_barrier(0);
      mma_dma(std::integral_constant<int, 1>{}, std::integral_constant<int, 2 * T::FN>{}, f1, wsc, asc);
      mx_load<BM, BN, AFP8, 3>(sw_of(buf), sa_of(buf), wn0, wm0, f1);
      __builtin_amdgcn_sched_barrier(0);
      mx_mma<BM, BN, AFP8, 2>(f0, wsc, asc, acc);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < T::FN; ++i) wsc3[i] = wsc[i];
#pragma unroll
      for (int jj = 0; jj < T::FM; ++jj) asc3[jj] = asc[jj];
      wait_lds_all();  // step-3 fragments are in registers
      wait_vmem_all();  // this wave's part of the next chunk landed
      __syncthreads();
      load_scales(buf ^ 1, wsc, asc);
      mx_load<BM, BN, AFP8, 0>(sw_of(buf ^ 1), sa_of(buf ^ 1), wn0, wm0, f0);
      __builtin_amdgcn_sched_barrier(0);
    }
    mx_mma<BM, BN, AFP8, 3>(f1, wsc3, asc3, acc);

    if (LR) {
      static_for<T::FN>([&](auto i) {
        static_for<T::FM>([&](auto jj) {
          acc[i][jj] = lowrank_block(p, acc[i][jj], cur.n0 + wn0 + 32 * i, cur.m0 + wm0 + 32 * jj);
        });
      });
    }
    if (staged_out) {
      // the buffer of the tile's last chunk is free: every wave read its step-3 fragments before
      // the last barrier, and the next tile's first load into it waits for the barrier below
      uint8_t* stage = smem + ((gc - 1) & 1) * T::STAGE + wave * (BM / 2) * 128;
      epilogue_staged<T::FN, T::FM, EPI, OUTF32>(p, acc, cur.n0 + wn0, cur.m0 + wm0, stage);
      __syncthreads();
    } else {
      epilogue_direct<T::FN, T::FM, EPI, OUTF32>(p, acc, cur.n0 + wn0, cur.m0 + wm0);
    }
    if (!has_next) break;
    j = jn;
    cur = nxt;
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
// low-rank down projection u = bf16(x . down_t^T): one wave per 32 (r) x 32 (m) block
// ---------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(64) lowrank_down_kernel(const uint16_t* __restrict__ x,
                                                           int64_t ld_x,
                                                           const uint16_t* __restrict__ down_t,
                                                           int M, int K, int R,
                                                           uint16_t* __restrict__ u) {
  const int lane = threadIdx.x;
  const int h = lane >> 5;
  const int rb = blockIdx.y * 32, mb = blockIdx.x * 32;
  const int r = min(rb + (lane & 31), R - 1);
  const int m = min(mb + (lane & 31), M - 1);
  v16f acc = v16f{};
  for (int k = 0; k < K; k += 16) {
    const uint4 da = *(const uint4*)(down_t + (int64_t)r * K + k + 8 * h);
    const uint4 xb = *(const uint4*)(x + (int64_t)m * ld_x + k + 8 * h);
    v8bf fa, fb;
    __builtin_memcpy(&fa, &da, 16);
    __builtin_memcpy(&fb, &xb, 16);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc, 0, 0, 0);
  }
  const int mo = mb + (lane & 31);
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
// Workgroups of the persistent GEMM launch: one per compute unit of the current device.
static int persistent_grid() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

template <int BM, int BN, bool AFP8, int EPI, bool OUTF32, bool LR>
static void run_mx_dma(const GemmParams& p, int grid, hipStream_t s) {
  gemm_mx_dma_kernel<BM, BN, AFP8, EPI, OUTF32, LR><<<grid, 256, 0, s>>>(p);
}

// The specialised instantiations: every epilogue for W4A4, the plain one (with and without the
// low-rank branch) for W4A8 and for W4A4 SVDQuant.  Other combinations take the generic kernel.
template <int BM, int BN, bool AFP8>
static bool run_mx_dma_epi(const GemmParams& p, int grid, hipStream_t s) {
  const bool lr = p.R > 0;
  if (p.epi == EPI_BIAS) {
    if (lr) {
      if (p.out_f32) run_mx_dma<BM, BN, AFP8, EPI_BIAS, true, true>(p, grid, s);
      else run_mx_dma<BM, BN, AFP8, EPI_BIAS, false, true>(p, grid, s);
    } else {
      if (p.out_f32) run_mx_dma<BM, BN, AFP8, EPI_BIAS, true, false>(p, grid, s);
      else run_mx_dma<BM, BN, AFP8, EPI_BIAS, false, false>(p, grid, s);
    }
    return true;
  }
  if constexpr (!AFP8) {
    if (lr) return false;
    if (p.epi == EPI_GELU_QUANT) run_mx_dma<BM, BN, AFP8, EPI_GELU_QUANT, false, false>(p, grid, s);
    else if (p.out_f32) run_mx_dma<BM, BN, AFP8, EPI_GELU, true, false>(p, grid, s);
    else run_mx_dma<BM, BN, AFP8, EPI_GELU, false, false>(p, grid, s);
    return true;
  }
  return false;
}

template <int BM, int BN, bool AFP8>
static hipError_t run_mx(const GemmParams& p, hipStream_t s) {
  const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  bool done = false;
  if (p.K % KC == 0) {
    const int cap = persistent_grid();
    const int grid = tiles < cap ? tiles : cap;
    done = run_mx_dma_epi<BM, BN, AFP8>(p, grid, s);
  }
  if (!done) gemm_mx_kernel<BM, BN, AFP8, false><<<tiles, 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_gemm_mx(const GemmParams& p, bool act_fp8, hipStream_t s) {
  if (p.M == 0) return hipSuccess;
  if (act_fp8) return run_mx<128, 256, true>(p, s);
  return run_mx<256, 256, false>(p, s);
}

hipError_t launch_gemm_nv(const GemmParams& p, hipStream_t s) {
  if (p.M == 0) return hipSuccess;
  const int tiles = ((p.M + 255) / 256) * ((p.N + 255) / 256);
  gemm_nv_kernel<256, 256><<<tiles, 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_lowrank_down(const uint16_t* x, int64_t ld_x, const uint16_t* down_t, int M,
                               int K, int R, uint16_t* u, hipStream_t s) {
  if (M == 0) return hipSuccess;
  dim3 grid((M + 31) / 32, (R + 31) / 32);
  lowrank_down_kernel<<<grid, 64, 0, s>>>(x, ld_x, down_t, M, K, R, u);
  return hipGetLastError();
}

}  // namespace mxk
