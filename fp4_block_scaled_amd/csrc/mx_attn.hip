// Microscaled attention for gfx950: the FP4 attention backend named by the MXFP4 Wan2.2 model
// cards (intel-ai/Wan2.2-I2V-A14B-Lightning-Diffusers-MXFP4-AutoRound, attention backends and
// Performance Profile), in the formats of the linear layer.  Q and K rows are MXFP4 along the
// head dimension (the activation quantizer's row-major output); V is MXFP8 along the key axis,
// stored transposed; the probabilities of each block are quantized to MXFP8 per 32 keys before
// they multiply V.  Both products run on V_MFMA_SCALE_F32_32X32X64_F8F6F4, so every MX scale is
// applied by the matrix core.
//
// Queries and keys may come from sequences of different lengths (Sq query rows, Skv key / value
// rows per head: self-attention, or the cross-attention of the DiT's second attention layer).
// Per block of 64 keys, with c = softmax_scale * log2(e):
//   s_j = c (q . k_j) (keys past Skv masked to -inf), m' = max(m, max_j s_j), alpha = 2^(m - m'),
//   p_j = 2^(s_j - m'), l = alpha l + sum_j p_j, o = alpha o + sum_j Q_MX8(p)_j v_j;
// the output is o / l.  The running maximum is exact (no deferred rescaling), so the quantized
// probabilities are the ones that definition gives; o is rescaled only when some query's maximum
// moved (alpha == 1 otherwise, and multiplying by it changes nothing).
#include <algorithm>

#include "mx_common.h"
#include "mx_internal.h"

namespace mxk {

constexpr int AT_D = 128;    // head dimension
constexpr int AT_KVB = 64;   // keys per block
constexpr int AT_WAVES = 4;  // waves per workgroup, 32 queries each

typedef short s16x2a __attribute__((ext_vector_type(2)));

// Combine a value with the one in lane ^ 32 (the other half of the wave).  V_PERMLANE32_SWAP
// exchanges the upper 32 lanes of its first register with the lower 32 lanes of its second; of a
// register with itself, the first result then holds the lower half's value in every lane and the
// second the upper half's, so both halves compute the same max or sum of the same two operands.
// max of three floats without the NaN-quieting moves the compiler adds before a library max in
// IEEE mode (the values here are finite scores or -inf, never NaN)
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float halves_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max3_raw(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------------------------
// V^T MXFP8 quantizer
// ---------------------------------------------------------------------------------------------
// Output in key blocks of 64: codes [BH, Sp / 64, D, 64] and scales [BH, Sp / 64, D, 2], so that
// one block of V^T (the 64 keys x D codes and 2 x D scales the attention kernel stages at a time)
// is contiguous.  A workgroup takes one unit (64 keys, 128 head-dim columns, one head) at a
// time: the BF16 tile is staged in LDS as loaded (key rows), then thread (d, g) gathers key group
// g of column d and quantizes it with the MXFP8 group routine of the activation quantizer.  Keys
// past S are zero.  Units are numbered heads first, then column tiles, then key blocks: with the
// heads of a token interleaved in memory ([B, S, H, D] activations), the workgroups in flight at
// once read whole contiguous token rows rather than one 256-byte piece of each (measured 2.5 %
// faster than key blocks first at 75600 x 40 x 128).  The grid walks the units with a stride of
// its size; the unit index is uniform in the workgroup, so every thread reaches the same barriers.
constexpr int VT_PITCH = 136;  // BF16 elements per LDS key row (272 bytes, 16-byte aligned)

__global__ __launch_bounds__(256) void quant_vt_kernel(const uint16_t* __restrict__ v, int64_t BH, int64_t S,
                                                       int64_t D, int64_t ld, int64_t hs, int64_t Sp,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[AT_KVB * VT_PITCH];
  const int64_t nkb = Sp / AT_KVB, ny = (D + 127) >> 7, units = nkb * ny * BH;
  const int d = threadIdx.x & 127, g = threadIdx.x >> 7;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const int64_t rest = u / BH, bh = u - rest * BH;
    const int64_t kb = rest / ny, d0 = (rest - kb * ny) * 128, kb0 = kb * AT_KVB;
    const int dn = (int)min((int64_t)128, D - d0);  // a multiple of 32
    const uint16_t* vb = v + bh * hs + d0;
    __syncthreads();  // the previous unit's gathers are done with the tile
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = threadIdx.x + 256 * i;  // 16-byte chunk: key row c / 16, columns 8 (c % 16)..
      const int r = c >> 4, cc = c & 15;
      uint4 x = make_uint4(0u, 0u, 0u, 0u);
      if (kb0 + r < S && 8 * cc < dn) x = *(const uint4*)(vb + (kb0 + r) * ld + 8 * cc);
      *(uint4*)(tile + r * VT_PITCH + 8 * cc) = x;
    }
    __syncthreads();
    if (d >= dn) continue;
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      w[i] = (uint32_t)tile[(32 * g + 2 * i) * VT_PITCH + d] |
             (uint32_t)tile[(32 * g + 2 * i + 1) * VT_PITCH + d] << 16;
    uint32_t out[8], sb;
    quant_fp8_group32(w, out, sb);
    const int64_t row = (bh * nkb + kb) * D + d0 + d;  // [BH, Sp / 64, D] rows
    uint4* dst = (uint4*)(codes + row * AT_KVB + 32 * g);
    dst[0] = uint4{out[0], out[1], out[2], out[3]};
    dst[1] = uint4{out[4], out[5], out[6], out[7]};
    scales[row * 2 + g] = (uint8_t)sb;
  }
}

hipError_t launch_quant_vt(const uint16_t* v, int64_t BH, int64_t S, int64_t D, int64_t ld, int64_t hs,
                           uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t Sp = (S + AT_KVB - 1) / AT_KVB * AT_KVB;
  const int64_t units = (Sp / AT_KVB) * ((D + 127) / 128) * BH;
  if (units == 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<int64_t>(units, 1 << 20);
  hipLaunchKernelGGL(quant_vt_kernel, dim3(grid), dim3(256), 0, s, v, BH, S, D, ld, hs, Sp, codes, scales);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// attention
// ---------------------------------------------------------------------------------------------
// Operand placement (see the GEMM kernels for the scaled MFMA's lane layout):
//  - scores: first operand K (32 keys), second Q (32 queries), K dimension the head dimension
//    (128 = two MFMAs, step s taking 32-element blocks 2h + s in the lanes of half h).  A lane
//    holds query l % 32 and, of each 32-key tile, keys 8 (e / 4) + 4 h + e % 4 (h = l / 32,
//    e = 0..15);
//  - PV: first operand V^T (32 head-dim rows), second the quantized probabilities (32 queries),
//    K dimension the 64 keys of the block (scale block b = keys 32 b..32 b + 31).  The FP8 operand
//    lane of half h must hold keys 16 h..16 h + 15 of each scale block: each lane has four runs
//    of 4 keys per tile (one dword of codes each) and trades two of them with lane ^ 32
//    (V_PERMLANE32_SWAP);
//  - the output tile has the scores' layout with head-dim rows in place of keys.
//
// A workgroup of 4 waves takes 128 queries of one head and walks the keys in blocks of 64
// through a 3-stage LDS ring: block b + 2 is fetched by direct-to-LDS buffer loads while block b
// is used, and each wave waits (vmcnt) only for its own loads of block b + 1 before the barrier
// that publishes it.  Stage: K codes (64 rows of 64 bytes), V^T codes (128 rows of 64 bytes),
// K scales (64 dwords), V^T scales (128 x 2 bytes).  Code rows hold their four 16-byte pieces
// XOR-swizzled by (row >> 2) & 3, so the 16 rows that a quarter wave reads at one piece index
// fall in distinct bank groups.
constexpr int AT_STAGES = 3;
constexpr int AT_KC = 64 * 64, AT_VC = AT_D * 64, AT_KS = 64 * 4, AT_VS = AT_D * 2;
constexpr int AT_STAGE = AT_KC + AT_VC + AT_KS + AT_VS;

template <int N>
__device__ __forceinline__ void at_wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void at_barrier() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ int at_swz(int row, int piece) { return row * 64 + 16 * (piece ^ ((row >> 2) & 3)); }

// Q_MX8 of one lane's 16 probabilities of a 32-key group whose (group-wide) maximum is amax >= 0:
// scale byte floor(log2 amax) - 8 (clamped to -127), magnitudes saturated at 448 * 2^e, then the
// scaled conversion, round to nearest even.  d[j] packs keys 4j..4j+3 of the lane's elements.
// Saturation: every p lies in [0, 512 * 2^e), and the conversion turns the ones that round past
// 448 * 2^e (E4M3 has no infinity) into the NaN byte 0x7F, which is rewritten to 0x7E, the code
// of 448: three integer operations per four codes instead of a clamp on every input.
__device__ __forceinline__ void quant_p8(const v16f& p, float amax, uint32_t (&d)[4], uint32_t& sb) {
  int e = (int)(__float_as_uint(amax) >> 23) - 127 - 8;
  if (e < -127) e = -127;
  const float scale = __uint_as_float(e >= -126 ? (uint32_t)(127 + e) << 23 : 0x00400000u);
  // both 16-bit halves of each result are written, so the first conversion's pass-through
  // operand (tied to its destination) is the first input, which dies there: no zeroing
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a0 = p[4 * j];
    s16x2a init;
    __builtin_memcpy(&init, &a0, 4);
    s16x2a r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(init, a0, p[4 * j + 1], scale, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, p[4 * j + 2], p[4 * j + 3], scale, true);
    uint32_t v;
    __builtin_memcpy(&v, &r, 4);
    // codes are at most 0x7F, so adding 1 to every byte carries into bit 7 exactly for 0x7F
    d[j] = v ^ (((v + 0x01010101u) >> 7) & 0x01010101u);
  }
  sb = (uint32_t)(e + 127);
}

template <bool OUTF32>
__global__ __launch_bounds__(64 * AT_WAVES, 2) void attn_mx_kernel(
    const uint8_t* __restrict__ qc, const uint8_t* __restrict__ qs, const uint8_t* __restrict__ kc,
    const uint8_t* __restrict__ ks, const uint8_t* __restrict__ vc, const uint8_t* __restrict__ vs,
    int Sq, int Skv, int nblk, int64_t ld_q, int64_t hs_q, int64_t ld_k, int64_t hs_k, float cexp,
    void* __restrict__ out, int64_t ld_o, int64_t hs_o) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[AT_STAGES * AT_STAGE];
  const int lane = lane_id(), r32 = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t bh = blockIdx.y;
  const int q = blockIdx.x * (32 * AT_WAVES) + wave * 32 + r32;
  const int64_t crow = ld_k / 2, srow = ld_k / 32;  // bytes per key row of codes / scales

  const int qr = min(q, Sq - 1);
  const uint8_t* qrow = qc + bh * (hs_q / 2) + qr * (ld_q / 2);
  const v4i qf0 = *(const v4i*)(qrow + 32 * h);
  const v4i qf1 = *(const v4i*)(qrow + 32 * h + 16);
  const uint32_t qsc = *(const uint32_t*)(qs + bh * (hs_q / 32) + qr * (ld_q / 32)) >> (16 * h);
  wait_vmem_all();  // from here on the only vector-memory loads in flight are the ring's

  // ring fill: per block, wave w loads K rows 16w..16w+15 and V^T rows 32w..32w+31 (1 KB per
  // instruction, lane i -> 16-byte slot i), wave 0 the K scales and wave 1 the V^T scales
  const v4i rk = make_rsrc_sgpr(kc + bh * (hs_k / 2), (uint32_t)((Skv - 1) * crow + 64));
  const v4i rks = make_rsrc_sgpr(ks + bh * (hs_k / 32), (uint32_t)((Skv - 1) * srow + 4));
  const v4i rv = make_rsrc_sgpr(vc + bh * (int64_t)nblk * AT_VC, (uint32_t)nblk * AT_VC);
  const v4i rvs = make_rsrc_sgpr(vs + bh * (int64_t)nblk * AT_VS, (uint32_t)nblk * AT_VS);
  const uint32_t lds0 = lds_addr_of(smem);
  const int krow = 16 * wave + (lane >> 2);
  const int kpiece = (lane & 3) ^ ((krow >> 2) & 3);
  const int vrow0 = 32 * wave + (lane >> 2), vrow1 = vrow0 + 16;
  const uint32_t voff0 = (uint32_t)(vrow0 * 64 + 16 * ((lane & 3) ^ ((vrow0 >> 2) & 3)));
  const uint32_t voff1 = (uint32_t)(vrow1 * 64 + 16 * ((lane & 3) ^ ((vrow1 >> 2) & 3)));
  // K byte offsets: row min(64 b + krow, Skv - 1) (rows past Skv are fetched but masked) as a
  // block offset plus loop-invariant per-lane parts, all below 2^32 (checked by the caller)
  const uint32_t koff = (uint32_t)(krow * crow + 16 * kpiece), kmax = (uint32_t)((Skv - 1) * crow + 16 * kpiece);
  const uint32_t ksoff = (uint32_t)(lane * srow), ksmax = (uint32_t)((Skv - 1) * srow);
  auto issue = [&](int b, int stage) {
    const uint32_t sb = lds0 + (uint32_t)(stage * AT_STAGE);
    const uint32_t kblk = (uint32_t)b * (uint32_t)(AT_KVB * crow);
    dma_lds16(rk, sb + (uint32_t)(wave * 1024), min(kblk + koff, kmax), 0u);
    dma_lds16(rv, sb + (uint32_t)(AT_KC + wave * 2048), voff0, (uint32_t)(b * AT_VC));
    dma_lds16(rv, sb + (uint32_t)(AT_KC + wave * 2048 + 1024), voff1, (uint32_t)(b * AT_VC));
    if (wave == 0) {
      const uint32_t sblk = (uint32_t)b * (uint32_t)(AT_KVB * srow);
      dma_lds4(rks, sb + (uint32_t)(AT_KC + AT_VC), min(sblk + ksoff, ksmax), 0u);
    } else if (wave == 1) {
      dma_lds4(rvs, sb + (uint32_t)(AT_KC + AT_VC + AT_KS), (uint32_t)(4 * lane), (uint32_t)(b * AT_VS));
    }
  };
  // this wave's loads of one block are complete when at most one block's worth is in flight
  auto wait_block = [&]() {
    if (wave < 2) at_wait_vmcnt<4>(); else at_wait_vmcnt<3>();
  };

  v16f o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dt][e] = 0.0f;
  float m = -__builtin_inff(), l = 0.0f;

  issue(0, 0);
  issue(min(1, nblk - 1), 1);
  wait_block();
  at_barrier();

  // One key block; the ring stage is a compile-time constant (the loop below is unrolled by the
  // ring depth), so every LDS address is a fixed offset from loop-invariant registers.
  auto step = [&](int b, auto stage_c) {
    constexpr int cur = decltype(stage_c)::value;
    // the last iterations refetch the last block into stages nobody reads again: every iteration
    // issues the same loads, so the wait below counts the same for all of them
    issue(min(b + 2, nblk - 1), (cur + 2) % AT_STAGES);
    const uint8_t* st = smem + cur * AT_STAGE;

    // scores
    v16f sc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int row = 32 * t + r32;
      const v4i k0 = *(const v4i*)(st + at_swz(row, 2 * h));
      const v4i k1 = *(const v4i*)(st + at_swz(row, 2 * h + 1));
      const int ksc = (int)(*(const uint32_t*)(st + AT_KC + AT_VC + 4 * row) >> (16 * h));
      v16f z;
#pragma unroll
      for (int e = 0; e < 16; ++e) z[e] = 0.0f;
      z = mfma_scale_32x32x64_f4f4(k0, qf0, z, 4, 4, 0, ksc, 0, (int)qsc);
      sc[t] = mfma_scale_32x32x64_f4f4(k1, qf1, z, 4, 4, 1, ksc, 1, (int)qsc);
    }
    // V^T fragments (read early: the softmax below covers their latency)
    v8i vf[4];
    int vsc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int row = 32 * dt + r32;
      const uint4 a = *(const uint4*)(st + AT_KC + at_swz(row, h));
      const uint4 c = *(const uint4*)(st + AT_KC + at_swz(row, 2 + h));
      vf[dt] = v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)c.x, (int)c.y, (int)c.z, (int)c.w};
      vsc[dt] = st[AT_KC + AT_VC + AT_KS + 2 * row + h];
    }

    // Keys past S are masked.  The running reference m' sits just below c * max(acc), and
    // p = 2^(c * acc - m') is evaluated with one fused multiply-add and clamped to [0, 1]: the
    // maximal key's exponent is >= 0 and tiny, so its p is exactly 1 as in the definition (a p
    // slightly below 1 would move its group's scale down a power of two).  Every p of a row
    // carries the same factor 2^(c * max - m'), which cancels in o / l.  The per-tile maxima of
    // acc give each 32-key group's largest p by the same expression.
    if ((b + 1) * AT_KVB > Skv) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (b * AT_KVB + 32 * t + 8 * (e >> 2) + 4 * h + (e & 3) >= Skv) sc[t][e] = -__builtin_inff();
    }
    float mt[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float x = max3_raw(sc[t][0], sc[t][1], sc[t][2]);
#pragma unroll
      for (int e = 3; e < 15; e += 2) x = max3_raw(x, sc[t][e], sc[t][e + 1]);
      mt[t] = halves_max(max3_raw(x, sc[t][15], sc[t][15]));
    }
    const float amx = max3_raw(mt[0], mt[1], mt[1]);  // finite: every block holds a key < Skv
    // mb = fp32(c * amx) lowered by |mb| 2^-23 (at least one ulp): strictly below the exact
    // c * amx for any normal mb, so the maximal key's exponent is >= 0 (a subnormal mb means
    // |c * amx| < 2^-126, where 2^exponent rounds to 1 anyway)
    const float mb0 = amx * cexp;
    const float mb = __builtin_fmaf(-__builtin_fabsf(mb0), 0x1p-23f, mb0);
    const float mn = max3_raw(m, mb, mb);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    float ps;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        // the clamp to [0, 1] is the exponential's output clamp modifier
        const float p = __builtin_amdgcn_fmed3f(__builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][e], cexp, -mn)), 0.0f, 1.0f);
        sc[t][e] = p;
        ps = (t == 0 && e == 0) ? p : ps + p;
      }
    l = l * alpha + ps;

    // Q_MX8 of the probabilities, then the PV operand: half 0 takes keys 0..15 of each tile,
    // half 1 keys 16..31.  Dword j of a lane holds keys 8j + 4h..8j + 4h + 3; V_PERMLANE32_SWAP
    // trades the upper half's dword 0 (1) for the lower half's dword 2 (3), which leaves both
    // halves with their 16 keys in order as dwords 0, 2, 1, 3.
    v8i pf;
    uint32_t psb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float gmax =  // = max of the group's p
          __builtin_amdgcn_fmed3f(__builtin_amdgcn_exp2f(__builtin_fmaf(mt[t], cexp, -mn)), 0.0f, 1.0f);
      uint32_t dw[4];
      quant_p8(sc[t], gmax, dw, psb[t]);
      const auto s02 = __builtin_amdgcn_permlane32_swap(dw[0], dw[2], false, false);
      const auto s13 = __builtin_amdgcn_permlane32_swap(dw[1], dw[3], false, false);
      pf[4 * t + 0] = (int)s02[0];
      pf[4 * t + 1] = (int)s02[1];
      pf[4 * t + 2] = (int)s13[0];
      pf[4 * t + 3] = (int)s13[1];
    }
    const int psc = (int)(h ? psb[1] : psb[0]);

    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      o[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[dt], pf, o[dt], 0, 0, 0, vsc[dt], 0, psc);

    wait_block();  // block b + 1 is in this wave's part of the ring
    at_barrier();
  };
  for (int b = 0; b < nblk; b += AT_STAGES) {
    step(b, std::integral_constant<int, 0>{});
    if (b + 1 < nblk) step(b + 1, std::integral_constant<int, 1>{});
    if (b + 2 < nblk) step(b + 2, std::integral_constant<int, 2>{});
  }
  static_assert(AT_STAGES == 3, "the block loop is unrolled by the ring depth");
  wait_vmem_all();  // the refetches of the last iterations land before the workgroup ends

  l = halves_sum(l);
  const float inv = 1.0f / l;
  if (q >= Sq) return;
  if (OUTF32) {
    float* orow = (float*)out + bh * hs_o + (int64_t)q * ld_o;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *(float4*)(orow + 32 * dt + 8 * j + 4 * h) =
            float4{o[dt][4 * j] * inv, o[dt][4 * j + 1] * inv, o[dt][4 * j + 2] * inv, o[dt][4 * j + 3] * inv};
  } else {
    uint16_t* orow = (uint16_t*)out + bh * hs_o + (int64_t)q * ld_o;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *(uint2*)(orow + 32 * dt + 8 * j + 4 * h) =
            uint2{pack_bf16x2(o[dt][4 * j] * inv, o[dt][4 * j + 1] * inv),
                  pack_bf16x2(o[dt][4 * j + 2] * inv, o[dt][4 * j + 3] * inv)};
  }
}

hipError_t launch_attn_mx(const uint8_t* qc, const uint8_t* qs, int64_t ld_q, int64_t hs_q, const uint8_t* kc,
                          const uint8_t* ks, int64_t ld_k, int64_t hs_k, const uint8_t* vc, const uint8_t* vs,
                          int64_t BH, int64_t Sq, int64_t Skv, float softmax_scale, bool out_f32, void* out,
                          int64_t ld_o, int64_t hs_o, hipStream_t s) {
  const int nblk = (int)((Skv + AT_KVB - 1) / AT_KVB);
  const float cexp = (float)((double)softmax_scale * 1.4426950408889634);  // softmax_scale * log2(e)
  dim3 grid((unsigned)((Sq + 32 * AT_WAVES - 1) / (32 * AT_WAVES)), (unsigned)BH);
  if (out_f32)
    hipLaunchKernelGGL(attn_mx_kernel<true>, grid, dim3(64 * AT_WAVES), 0, s, qc, qs, kc, ks, vc, vs, (int)Sq,
                       (int)Skv, nblk, ld_q, hs_q, ld_k, hs_k, cexp, out, ld_o, hs_o);
  else
    hipLaunchKernelGGL(attn_mx_kernel<false>, grid, dim3(64 * AT_WAVES), 0, s, qc, qs, kc, ks, vc, vs, (int)Sq,
                       (int)Skv, nblk, ld_q, hs_q, ld_k, hs_k, cexp, out, ld_o, hs_o);
  return hipGetLastError();
}

}  // namespace mxk
