// moe_device.h -- device helpers of the gfx950 kernels: bf16 / fp32 staging
// of activations, the dequantising row dots, top-K selection, router rows and
// the gate/up and down tiles; host-side tile geometry.  Included by the kernel
// translation units only.
#pragma once

#include "moe_internal.h"
#include "moe_sortnet.h"

#include <math.h>
#include <stdint.h>

#include <type_traits>

namespace moe_impl {

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__host__ __device__ __forceinline__ int ceil_log2(int v) {
  return v <= 1 ? 0 : 32 - __builtin_clz((unsigned)(v - 1));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Sum over aligned groups of 2^lg lanes; every lane of a group gets the sum.
__device__ __forceinline__ float seg_sum(float v, int lg) {
  if (lg >= 1) v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  if (lg >= 2) v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  if (lg >= 3) v += dpp<0x141>(v);  // row_half_mirror
  if (lg >= 4) v += dpp<0x140>(v);  // row_mirror
  if (lg >= 5) v += __shfl_xor(v, 16, 64);
  if (lg >= 6) v += __shfl_xor(v, 32, 64);
  return v;
}

__device__ __forceinline__ float silu_mul(float a, float u) { return a / (1.0f + expf(-a)) * u; }

// hide a value's provenance from the optimiser (no instruction is emitted)
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// ---------------------------------------------------------------------------
// staged input chunk: what one lane keeps of x for one 16-byte code chunk
// ---------------------------------------------------------------------------
// A 4-bit chunk covers 32 columns in 4 words: word t holds columns 8t..8t+7,
// column 8t+n at bits 4n.  A 2-bit chunk covers 64 columns: word t holds
// columns 16t..16t+15, column 16t+f at bits 2f.
//
// bf16 input (XF32 = false): the dot runs on v_dot2_f32_bf16.  A code is
//   moved to mantissa bits 3..6 of bf16 16.0 (0x4180), which makes the bf16
//   number 16 + q (a 2-bit field at bits 5..6 gives 16 + 4q, met by x/4).
//   Products are exact in fp32; the constant 16 * x part ("off", computed at
//   staging with the same instruction) is removed through the accumulator's
//   start value.  With the code at the top of the mantissa the constant part
//   stays small next to q * x, so little precision is lost to cancellation.
//   4-bit pair 4t+n = (x[8t+n], x[8t+4+n]): nibble n of each 16-bit half.
//   2-bit pair 8t+f = (x[16t+f], x[16t+8+f]) * (f odd ? 1/4 : 1).
// fp32 input (XF32 = true): codes become fp32 through the byte converts
//   (v_cvt_f32_ubyte0..3 of nibble- or field-masked words) and meet x in fp32
//   FMAs, so nothing of x is rounded.
template <int BITS>
struct ChunkGeom {
  static constexpr int kCols = 128 / BITS;        // columns per 16-byte chunk
  static constexpr int kPairs = kCols / 2;
};

constexpr uint32_t kMagic16 = 0x41804180u;  // two bf16 16.0

template <int BITS, bool XF32>
struct XStage;

template <int BITS>
struct XStage<BITS, false> {
  uint32_t p[ChunkGeom<BITS>::kPairs];
  float off;  // sum over the chunk of 16 * x' (the constant part of the codes)
  float xs;   // sum of x over the chunk (multiplies the group bias)
};

template <int BITS>
struct XStage<BITS, true> {
  float v[ChunkGeom<BITS>::kCols];
  float xs;
};

template <int BITS>
__device__ __forceinline__ void stage_chunk(const float (&v)[ChunkGeom<BITS>::kCols],
                                            XStage<BITS, false> &s) {
  constexpr int NC = ChunkGeom<BITS>::kCols;
  constexpr int CPW = NC / 4;                        // columns per word
  constexpr int PPW = ChunkGeom<BITS>::kPairs / 4;   // pairs per word
  float xs = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) xs += v[c];
  s.xs = xs;
  float off = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
      const float sc = (BITS == 2 && (j & 1)) ? 0.25f : 1.0f;
      const uint32_t ha = bf16_rne(v[CPW * t + j] * sc);
      const uint32_t hb = bf16_rne(v[CPW * t + CPW / 2 + j] * sc);
      const uint32_t hp = ha | (hb << 16);
      s.p[PPW * t + j] = hp;
      off = dot2bf(kMagic16, hp, off);
    }
  }
  s.off = off;
}

template <int BITS>
__device__ __forceinline__ void stage_chunk(const float (&v)[ChunkGeom<BITS>::kCols],
                                            XStage<BITS, true> &s) {
  constexpr int NC = ChunkGeom<BITS>::kCols;
  float xs = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    s.v[c] = v[c];
    xs += v[c];
  }
  s.xs = xs;
}

// the codes of one 16-byte chunk as the bf16 pairs chunk_dot2 forms (16 + q,
// or 16 + 4q for the odd 2-bit fields), in the staged pairs' order
template <int BITS>
__device__ __forceinline__ void chunk_pairs(const uint4 &q, uint32_t magic,
                                            uint32_t (&pr)[ChunkGeom<BITS>::kPairs]) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t a3 = w[t] << 3, a1 = w[t] >> 1, a5 = w[t] >> 5, a9 = w[t] >> 9;
    if constexpr (BITS == 4) {
      constexpr uint32_t M = 0x00780078u;
      pr[4 * t + 0] = (a3 & M) | magic;
      pr[4 * t + 1] = (a1 & M) | magic;
      pr[4 * t + 2] = (a5 & M) | magic;
      pr[4 * t + 3] = (a9 & M) | magic;
    } else {
      constexpr uint32_t L = 0x00180018u, Hm = 0x00600060u;
      pr[8 * t + 0] = (a3 & L) | magic;
      pr[8 * t + 1] = (a3 & Hm) | magic;
      pr[8 * t + 2] = (a1 & L) | magic;
      pr[8 * t + 3] = (a1 & Hm) | magic;
      pr[8 * t + 4] = (a5 & L) | magic;
      pr[8 * t + 5] = (a5 & Hm) | magic;
      pr[8 * t + 6] = (a9 & L) | magic;
      pr[8 * t + 7] = (a9 & Hm) | magic;
    }
  }
}

// sum_c q_c * x_c over one 16-byte code chunk, for two chunks at once (two
// independent accumulation chains: gate and up, or two rows)
template <int BITS>
__device__ __forceinline__ void chunk_dot2(const uint4 &qa, const uint4 &qb,
                                           const XStage<BITS, false> &s, uint32_t magic,
                                           float &da, float &db) {
  float a = -s.off, b = -s.off;
  const uint32_t wa[4] = {qa.x, qa.y, qa.z, qa.w};
  const uint32_t wb[4] = {qb.x, qb.y, qb.z, qb.w};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t a3 = wa[t] << 3, a1 = wa[t] >> 1, a5 = wa[t] >> 5, a9 = wa[t] >> 9;
    const uint32_t b3 = wb[t] << 3, b1 = wb[t] >> 1, b5 = wb[t] >> 5, b9 = wb[t] >> 9;
    if constexpr (BITS == 4) {
      constexpr uint32_t M = 0x00780078u;
      a = dot2bf((a3 & M) | magic, s.p[4 * t + 0], a);
      b = dot2bf((b3 & M) | magic, s.p[4 * t + 0], b);
      a = dot2bf((a1 & M) | magic, s.p[4 * t + 1], a);
      b = dot2bf((b1 & M) | magic, s.p[4 * t + 1], b);
      a = dot2bf((a5 & M) | magic, s.p[4 * t + 2], a);
      b = dot2bf((b5 & M) | magic, s.p[4 * t + 2], b);
      a = dot2bf((a9 & M) | magic, s.p[4 * t + 3], a);
      b = dot2bf((b9 & M) | magic, s.p[4 * t + 3], b);
    } else {
      constexpr uint32_t L = 0x00180018u, Hm = 0x00600060u;
      a = dot2bf((a3 & L) | magic, s.p[8 * t + 0], a);
      b = dot2bf((b3 & L) | magic, s.p[8 * t + 0], b);
      a = dot2bf((a3 & Hm) | magic, s.p[8 * t + 1], a);
      b = dot2bf((b3 & Hm) | magic, s.p[8 * t + 1], b);
      a = dot2bf((a1 & L) | magic, s.p[8 * t + 2], a);
      b = dot2bf((b1 & L) | magic, s.p[8 * t + 2], b);
      a = dot2bf((a1 & Hm) | magic, s.p[8 * t + 3], a);
      b = dot2bf((b1 & Hm) | magic, s.p[8 * t + 3], b);
      a = dot2bf((a5 & L) | magic, s.p[8 * t + 4], a);
      b = dot2bf((b5 & L) | magic, s.p[8 * t + 4], b);
      a = dot2bf((a5 & Hm) | magic, s.p[8 * t + 5], a);
      b = dot2bf((b5 & Hm) | magic, s.p[8 * t + 5], b);
      a = dot2bf((a9 & L) | magic, s.p[8 * t + 6], a);
      b = dot2bf((b9 & L) | magic, s.p[8 * t + 6], b);
      a = dot2bf((a9 & Hm) | magic, s.p[8 * t + 7], a);
      b = dot2bf((b9 & Hm) | magic, s.p[8 * t + 7], b);
    }
  }
  da = a;
  db = b;
}

// fp32 input: the byte converts and fp32 FMAs, for two chunks (TWO) or for
// qa alone (the odd last row of a wave's passes: the masked words pass
// through an asm barrier, so a second chain over the same chunk would not be
// merged with the first and would cost its instructions again)
template <int BITS, bool TWO>
__device__ __forceinline__ void chunk_dot_f32(const uint4 &qa, const uint4 &qb,
                                              const XStage<BITS, true> &s, float &da, float &db) {
  float a = 0.f, b = 0.f;
  const uint32_t wa[4] = {qa.x, qa.y, qa.z, qa.w};
  const uint32_t wb[4] = {qb.x, qb.y, qb.z, qb.w};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if constexpr (BITS == 4) {
      // bytes of lo: nibbles 0,2,4,6; bytes of hi: nibbles 1,3,5,7
      const uint32_t la = opaque(wa[t] & 0x0F0F0F0Fu), ha = opaque((wa[t] >> 4) & 0x0F0F0F0Fu);
      uint32_t lb = 0, hb = 0;
      if constexpr (TWO) {
        lb = opaque(wb[t] & 0x0F0F0F0Fu);
        hb = opaque((wb[t] >> 4) & 0x0F0F0F0Fu);
      }
      const float *x = s.v + 8 * t;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t sh = 8 * k;
        const float xl = x[2 * k], xh = x[2 * k + 1];
        const uint32_t qla = k == 3 ? (la >> 24) : ((la >> sh) & 0xFFu);
        const uint32_t qha = k == 3 ? (ha >> 24) : ((ha >> sh) & 0xFFu);
        a = fmaf((float)qla, xl, a);
        if constexpr (TWO) {
          const uint32_t qlb = k == 3 ? (lb >> 24) : ((lb >> sh) & 0xFFu);
          b = fmaf((float)qlb, xl, b);
        }
        a = fmaf((float)qha, xh, a);
        if constexpr (TWO) {
          const uint32_t qhb = k == 3 ? (hb >> 24) : ((hb >> sh) & 0xFFu);
          b = fmaf((float)qhb, xh, b);
        }
      }
    } else {
      // byte bb of f_k is field 4*bb + k
      uint32_t fa[4], fb[4] = {0, 0, 0, 0};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        fa[k] = opaque((wa[t] >> (2 * k)) & 0x03030303u);
        if constexpr (TWO) fb[k] = opaque((wb[t] >> (2 * k)) & 0x03030303u);
      }
      const float *x = s.v + 16 * t;
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t qa8 = bb == 3 ? (fa[k] >> 24) : ((fa[k] >> (8 * bb)) & 0xFFu);
          a = fmaf((float)qa8, x[4 * bb + k], a);
          if constexpr (TWO) {
            const uint32_t qb8 = bb == 3 ? (fb[k] >> 24) : ((fb[k] >> (8 * bb)) & 0xFFu);
            b = fmaf((float)qb8, x[4 * bb + k], b);
          }
        }
      }
    }
  }
  da = a;
  db = b;
}

template <int BITS>
__device__ __forceinline__ void chunk_dot2(const uint4 &qa, const uint4 &qb,
                                           const XStage<BITS, true> &s, uint32_t,
                                           float &da, float &db) {
  chunk_dot_f32<BITS, true>(qa, qb, s, da, db);
}

// raw x of one chunk as loaded (bf16 words or fp32), before the staging math;
// loading and staging are separate so that other loads can be issued between
template <int BITS, int XS>
struct XRaw {
  static constexpr int kN = (XS == XS_BF16) ? ChunkGeom<BITS>::kCols / 8 : ChunkGeom<BITS>::kCols / 4;
  uint4 u[kN];
  float xs;  // XS_LDSPAD: the chunk's column sum, stored with it
};

template <int BITS, int XS>
__device__ __forceinline__ XRaw<BITS, XS> load_raw(const void *x, const float *xl, int c) {
  XRaw<BITS, XS> r;
  const int col0 = c * ChunkGeom<BITS>::kCols;
  const uint4 *p;
  if constexpr (XS == XS_BF16) p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + col0);
  else if constexpr (XS == XS_LDSPAD) p = reinterpret_cast<const uint4 *>(xl + c * (ChunkGeom<BITS>::kCols + kLdsPad));
  else p = reinterpret_cast<const uint4 *>(((XS == XS_F32) ? static_cast<const float *>(x) : xl) + col0);
#pragma unroll
  for (int i = 0; i < XRaw<BITS, XS>::kN; ++i) r.u[i] = p[i];
  if constexpr (XS == XS_LDSPAD) r.xs = xl[c * (ChunkGeom<BITS>::kCols + kLdsPad) + ChunkGeom<BITS>::kCols];
  return r;
}

template <int BITS, int XS>
__device__ __forceinline__ XStage<BITS, XS != XS_BF16> stage_raw(const XRaw<BITS, XS> &r) {
  if constexpr (BITS == 4 && XS == XS_BF16) {
    // bf16 x, 4-bit codes: pair 4t + n = (x[8t + n], x[8t + 4 + n]) is two
    // bf16 halves of the loaded words, gathered by one byte permute; the
    // sum of x is the constant part of the codes divided by 16 (exact
    // scaling of the same fp32 sum)
    XStage<4, false> s;
    float off = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint4 u = r.u[t];
      s.p[4 * t + 0] = __builtin_amdgcn_perm(u.z, u.x, 0x05040100u);
      s.p[4 * t + 1] = __builtin_amdgcn_perm(u.z, u.x, 0x07060302u);
      s.p[4 * t + 2] = __builtin_amdgcn_perm(u.w, u.y, 0x05040100u);
      s.p[4 * t + 3] = __builtin_amdgcn_perm(u.w, u.y, 0x07060302u);
#pragma unroll
      for (int n = 0; n < 4; ++n) off = dot2bf(kMagic16, s.p[4 * t + n], off);
    }
    s.off = off;
    s.xs = off * 0.0625f;
    return s;
  }
  float v[ChunkGeom<BITS>::kCols];
#pragma unroll
  for (int i = 0; i < XRaw<BITS, XS>::kN; ++i) {
    const uint4 u = r.u[i];
    if constexpr (XS == XS_BF16) {
      v[8 * i + 0] = bf_lo(u.x); v[8 * i + 1] = bf_hi(u.x);
      v[8 * i + 2] = bf_lo(u.y); v[8 * i + 3] = bf_hi(u.y);
      v[8 * i + 4] = bf_lo(u.z); v[8 * i + 5] = bf_hi(u.z);
      v[8 * i + 6] = bf_lo(u.w); v[8 * i + 7] = bf_hi(u.w);
    } else {
      v[4 * i + 0] = __uint_as_float(u.x); v[4 * i + 1] = __uint_as_float(u.y);
      v[4 * i + 2] = __uint_as_float(u.z); v[4 * i + 3] = __uint_as_float(u.w);
    }
  }
  XStage<BITS, XS != XS_BF16> s;
  if constexpr (XS == XS_LDSPAD) {
#pragma unroll
    for (int c = 0; c < ChunkGeom<BITS>::kCols; ++c) s.v[c] = v[c];
    s.xs = r.xs;
  } else {
    stage_chunk<BITS>(v, s);
  }
  return s;
}

// Store four columns of an fp32 activation into its LDS copy padded per code
// chunk (XS_LDSPAD) and the chunk's column sum after its columns.  The
// kCols / 4 consecutive lanes that hold one chunk call this together (the sum
// is a DPP reduction over them); col is the first of the four columns.
template <int BITS>
__device__ __forceinline__ void lds_put_chunk4(float *row, int col, const float4 &v) {
  constexpr int NC = ChunkGeom<BITS>::kCols;
  constexpr int LG = NC == 32 ? 3 : 4;  // log2 of the lanes per chunk
  const int chunk = col / NC;
  const int cc = col - chunk * NC;
  float *base = row + chunk * (NC + kLdsPad);
  *reinterpret_cast<float4 *>(base + cc) = v;
  const float sum = seg_sum((v.x + v.y) + (v.z + v.w), LG);
  if (cc == 0) base[NC] = sum;
}

// stage chunk c of x from x itself
template <int BITS, int XS>
__device__ __forceinline__ XStage<BITS, XS != XS_BF16> make_stage(const void *x, const float *xl,
                                                                  int c) {
  return stage_raw<BITS, XS>(load_raw<BITS, XS>(x, xl, c));
}

// chunk c of bf16 x as staged once into global memory (write_xstage)
template <int BITS>
__device__ __forceinline__ XStage<BITS, false> read_stage(const uint32_t *xs_pairs,
                                                          const float *xs_sums, int c) {
  constexpr int NP = ChunkGeom<BITS>::kPairs;
  XStage<BITS, false> s;
  const uint4 *pp = reinterpret_cast<const uint4 *>(xs_pairs + (size_t)c * NP);
#pragma unroll
  for (int i = 0; i < NP / 4; ++i) {
    const uint4 u = pp[i];
    s.p[4 * i + 0] = u.x;
    s.p[4 * i + 1] = u.y;
    s.p[4 * i + 2] = u.z;
    s.p[4 * i + 3] = u.w;
  }
  const float2 sm = reinterpret_cast<const float2 *>(xs_sums)[c];
  s.off = sm.x;
  s.xs = sm.y;
  return s;
}

// ---------------------------------------------------------------------------
// x staged once per workgroup in LDS (the gate/up kernel).  Each thread loads
// a slice of x, stages it into LDS, and after one barrier every wave reads
// the chunks its lanes need: x crosses from L2 once per workgroup instead of
// once per wave, and the bf16 staging math runs once per chunk.
//   bf16 x: chunk c holds its staged pairs, the constant part and the column
//           sum (kPairs + 2 words, rounded up to a multiple of 4 so that each
//           chunk starts 16-byte aligned); thread kBlock - 1 - c stages it
//           (2-bit: threads kBlock - 1 - 2c and kBlock - 2 - 2c, a half
//           each), so that wave 0 (which selects the experts) stages none
//           while the chunks fit in the other waves.
//   fp32 x: chunk c holds its columns, then kLdsPad floats of which the first
//           is the column sum (the XS_LDSPAD layout); thread t stores the
//           four columns 4t + 4 kBlock i.
// ---------------------------------------------------------------------------

template <int BITS, bool XF32>
struct XLds {
  static constexpr int kWords = XF32 ? ChunkGeom<BITS>::kCols + kLdsPad
                                     : (ChunkGeom<BITS>::kPairs + 2 + 3) / 4 * 4;
  static constexpr int kF4 = kMaxDim / (4 * kBlock);  // fp32: float4 per thread at most
  static_assert(kMaxDim * BITS / 128 <= kBlock, "one bf16 chunk per thread");
};

template <int BITS, int XS>
struct XPart;
template <int BITS>
struct XPart<BITS, XS_BF16> {
  XRaw<BITS, XS_BF16> r;
};
// 2-bit rows: a chunk's 64 bf16 columns are split over two threads (an
// aligned pair of lanes, 32 columns each), so a thread holds 16 registers of
// x through the selection instead of 32
template <>
struct XPart<2, XS_BF16> {
  uint4 u[4];
};
template <int BITS>
struct XPart<BITS, XS_F32> {
  float4 v[XLds<BITS, true>::kF4];
};

template <int BITS, int XS>
__device__ __forceinline__ void xpart_load(XPart<BITS, XS> &xp, const void *x, int H) {
  const int t = threadIdx.x;
  if constexpr (BITS == 2 && XS == XS_BF16) {
    // thread kBlock - 1 - (2 c + h) loads half h of chunk c
    const int cpr = H / ChunkGeom<2>::kCols;
    const int q = kBlock - 1 - t, c = q >> 1, h = q & 1;
    const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) +
                                                       (c < cpr ? c : 0) * ChunkGeom<2>::kCols + 32 * h);
#pragma unroll
    for (int i = 0; i < 4; ++i) xp.u[i] = src[i];
  } else if constexpr (XS == XS_BF16) {
    const int cpr = H / ChunkGeom<BITS>::kCols;
    const int c = kBlock - 1 - t;
    xp.r = load_raw<BITS, XS_BF16>(x, nullptr, c < cpr ? c : 0);
  } else {
    const float4 *xf = static_cast<const float4 *>(x);
#pragma unroll
    for (int i = 0; i < XLds<BITS, true>::kF4; ++i) {
      const int q = i * kBlock + t;  // float4 index
      xp.v[i] = xf[4 * q < H ? q : 0];
    }
  }
}

template <int BITS, int XS>
__device__ __forceinline__ void xpart_store(const XPart<BITS, XS> &xp, uint32_t *xw, int H,
                                            float scale = 1.0f) {
  const int t = threadIdx.x;
  if constexpr (BITS == 2 && XS == XS_BF16) {
    // Half h of a chunk is words 2h and 2h + 1 (columns 32h..32h + 31): its
    // 16 staged pairs (pair 8w + f = (x[16w + f], x[16w + 8 + f]), times 1/4
    // for odd f, the pairs stage_chunk forms) and its partial constant part
    // and column sum; the two halves' partials are added across the lane
    // pair (the same sum in both lanes: fp32 addition commutes).
    constexpr int NP = ChunkGeom<2>::kPairs;
    static_assert(2 * (kMaxDim / ChunkGeom<2>::kCols) <= kBlock, "two threads per 2-bit chunk");
    const int q = kBlock - 1 - t, c = q >> 1, h = q & 1;
    // Loaded word i of the half holds columns 2i (low) and 2i + 1 (high) of
    // it; pair 8w + f takes columns 16w + f and 16w + 8 + f, i.e. half f % 2
    // of words 8w + f / 2 and 8w + 4 + f / 2.  Even f: the two low halves as
    // they are (a byte permute).  Odd f: the two high halves times 1/4 (exact
    // in fp32 for |x| >= 2^-124), whose upper 16 bits are then the bf16
    // values (RNE of an exact value keeps them), gathered by a byte permute.
    const uint32_t *r = reinterpret_cast<const uint32_t *>(xp.u);
    uint32_t pr[16];
    float off_e = 0.f, off_o = 0.f;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t a = r[8 * w + j], b = r[8 * w + 4 + j];
        const uint32_t ev = __builtin_amdgcn_perm(b, a, 0x05040100u);
        const uint32_t qa = __float_as_uint(bf_hi(a) * 0.25f), qb = __float_as_uint(bf_hi(b) * 0.25f);
        const uint32_t od = __builtin_amdgcn_perm(qb, qa, 0x07060302u);
        pr[8 * w + 2 * j] = ev;
        pr[8 * w + 2 * j + 1] = od;
        off_e = dot2bf(kMagic16, ev, off_e);
        off_o = dot2bf(kMagic16, od, off_o);
      }
    }
    // the constant part is 16 x over the even pairs and 4 x over the odd
    // ones, so the column sum is (off_e + 4 off_o) / 16 (scalings by powers
    // of two)
    float off = off_e + off_o;
    float xs = (off_e + 4.0f * off_o) * 0.0625f;
    off += dpp<0xB1>(off);  // quad_perm [1,0,3,2]: the other half's partial
    xs += dpp<0xB1>(xs);
    if (c < H / ChunkGeom<2>::kCols) {
      uint32_t *d = xw + c * XLds<2, false>::kWords;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint4 *>(d + 16 * h + 4 * i) = make_uint4(pr[4 * i], pr[4 * i + 1], pr[4 * i + 2], pr[4 * i + 3]);
      if (h == 0) *reinterpret_cast<float2 *>(d + NP) = make_float2(off, xs);
    }
  } else if constexpr (XS == XS_BF16) {
    constexpr int NP = ChunkGeom<BITS>::kPairs;
    const int c = kBlock - 1 - t;
    if (c < H / ChunkGeom<BITS>::kCols) {
      const XStage<BITS, false> s = stage_raw<BITS, XS_BF16>(xp.r);
      uint32_t *d = xw + c * XLds<BITS, false>::kWords;
#pragma unroll
      for (int i = 0; i < NP / 4; ++i)
        *reinterpret_cast<uint4 *>(d + 4 * i) = make_uint4(s.p[4 * i], s.p[4 * i + 1], s.p[4 * i + 2], s.p[4 * i + 3]);
      *reinterpret_cast<float2 *>(d + NP) = make_float2(s.off, s.xs);
    }
  } else {
    float *xl = reinterpret_cast<float *>(xw);
#pragma unroll
    for (int i = 0; i < XLds<BITS, true>::kF4; ++i) {
      const int col = 4 * (i * kBlock + t);
      // H is a multiple of 64, so a chunk's lanes agree on col < H
      const float4 v = xp.v[i];
      if (col < H) lds_put_chunk4<BITS>(xl, col, make_float4(v.x * scale, v.y * scale, v.z * scale, v.w * scale));
    }
  }
}

// the staged chunk c as the dot products take it
template <int BITS, bool XF32>
__device__ __forceinline__ XStage<BITS, XF32> xlds_read(const uint32_t *xw, int c) {
  if constexpr (XF32) {
    return stage_raw<BITS, XS_LDSPAD>(load_raw<BITS, XS_LDSPAD>(nullptr, reinterpret_cast<const float *>(xw), c));
  } else {
    constexpr int NP = ChunkGeom<BITS>::kPairs;
    const uint32_t *d = xw + c * XLds<BITS, false>::kWords;
    XStage<BITS, false> s;
#pragma unroll
    for (int i = 0; i < NP / 4; ++i) {
      const uint4 u = *reinterpret_cast<const uint4 *>(d + 4 * i);
      s.p[4 * i + 0] = u.x;
      s.p[4 * i + 1] = u.y;
      s.p[4 * i + 2] = u.z;
      s.p[4 * i + 3] = u.w;
    }
    const float2 sm = *reinterpret_cast<const float2 *>(d + NP);
    s.off = sm.x;
    s.xs = sm.y;
    return s;
  }
}

// lane layout over rows of `cols` columns at BITS bits
struct RowMap {
  int cpr;      // 16-byte chunks per row
  int lg;       // log2(lanes per row)
  int rpp;      // rows per pass of the wave
  int li;       // lane index inside its row group
  int rip;      // row of this lane inside the pass
  int wpr;      // u32 words per row
  int gpr;      // groups per row
};

template <int BITS>
__device__ __forceinline__ RowMap row_map(int cols) {
  RowMap m;
  m.cpr = cols / ChunkGeom<BITS>::kCols;
  m.lg = ceil_log2(m.cpr);
  if (m.lg > 6) m.lg = 6;
  m.rpp = 64 >> m.lg;
  const int lane = lane_id();
  m.li = lane & ((1 << m.lg) - 1);
  m.rip = lane >> m.lg;
  m.wpr = cols * BITS / 32;
  m.gpr = cols / 64;
  return m;
}

template <int BITS>
__device__ __forceinline__ int chunk_group(int c) { return BITS == 4 ? (c >> 1) : c; }

// ---------------------------------------------------------------------------
// gate/up + SwiGLU ([openclawradar] "Metal compute shaders": fused SwiGLU;
// h = silu(a) * u with a = W_gate x, u = W_up x)
// ---------------------------------------------------------------------------
template <int BITS, int NCH, int NPASS>
struct GUTile {
  uint4 gq[NPASS][NCH], uq[NPASS][NCH];
  uint32_t gs[NPASS][NCH], us[NPASS][NCH];
};

// Every lane loads (row 0 / chunk 0 stand in for positions past the end, so
// each address is valid); what lies outside is masked where it is used.  With
// no branch or use next to them, the loads are all in flight before the first
// wait.
template <int BITS, int NCH, int NPASS>
__device__ __forceinline__ void gu_load(GUTile<BITS, NCH, NPASS> &t, const uint8_t *rec,
                                        const RecOffsets &off, const RowMap &m, int I, int row0) {
  const uint32_t *gc = reinterpret_cast<const uint32_t *>(rec + off.gate_codes);
  const uint32_t *uc = reinterpret_cast<const uint32_t *>(rec + off.up_codes);
  const uint32_t *gs = reinterpret_cast<const uint32_t *>(rec + off.gate_sb);
  const uint32_t *us = reinterpret_cast<const uint32_t *>(rec + off.up_sb);
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int r = row0 + p * m.rpp + m.rip;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = m.li + (j << m.lg);
      const bool in = r < I && c < m.cpr;
      const int rr = in ? r : 0, cc = in ? c : 0;
      const size_t wo = (size_t)rr * m.wpr + (size_t)cc * 4;
      const size_t so = (size_t)rr * m.gpr + chunk_group<BITS>(cc);
      t.gq[p][j] = *reinterpret_cast<const uint4 *>(gc + wo);
      t.uq[p][j] = *reinterpret_cast<const uint4 *>(uc + wo);
      t.gs[p][j] = gs[so];
      t.us[p][j] = us[so];
    }
  }
}

// the same words written back at the same offsets of another record (the
// expert tier's read-through fill of a cache slot; positions past the end
// rewrite row 0 / chunk 0 with what they read there)
template <int BITS, int NCH, int NPASS>
__device__ __forceinline__ void gu_store(const GUTile<BITS, NCH, NPASS> &t, uint8_t *rec,
                                         const RecOffsets &off, const RowMap &m, int I, int row0) {
  uint32_t *gc = reinterpret_cast<uint32_t *>(rec + off.gate_codes);
  uint32_t *uc = reinterpret_cast<uint32_t *>(rec + off.up_codes);
  uint32_t *gs = reinterpret_cast<uint32_t *>(rec + off.gate_sb);
  uint32_t *us = reinterpret_cast<uint32_t *>(rec + off.up_sb);
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int r = row0 + p * m.rpp + m.rip;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = m.li + (j << m.lg);
      const bool in = r < I && c < m.cpr;
      const int rr = in ? r : 0, cc = in ? c : 0;
      const size_t wo = (size_t)rr * m.wpr + (size_t)cc * 4;
      const size_t so = (size_t)rr * m.gpr + chunk_group<BITS>(cc);
      *reinterpret_cast<uint4 *>(gc + wo) = t.gq[p][j];
      *reinterpret_cast<uint4 *>(uc + wo) = t.uq[p][j];
      gs[so] = t.gs[p][j];
      us[so] = t.us[p][j];
    }
  }
}

__device__ __forceinline__ bool in_tile(const RowMap &m, int rows, int row0, int p, int j) {
  return row0 + p * m.rpp + m.rip < rows && m.li + (j << m.lg) < m.cpr;
}

template <int BITS, int NCH, int NPASS, bool XF32>
__device__ __forceinline__ void gu_compute(const GUTile<BITS, NCH, NPASS> &t,
                                           const XStage<BITS, XF32> (&xs)[NCH], const RowMap &m,
                                           int I, int row0, bool valid, float *h_out) {
  // the magic constant lives in a VGPR so that mask-and-or is one v_and_or_b32
  // (gfx9 VOP3 reads at most one scalar or literal operand)
  const uint32_t magic = opaque(kMagic16);
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    float a = 0.f, u = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      // positions past the end get zero scale and bias
      const bool in = in_tile(m, I, row0, p, j);
      const uint32_t gsw = in ? t.gs[p][j] : 0u, usw = in ? t.us[p][j] : 0u;
      float da, du;
      chunk_dot2<BITS>(t.gq[p][j], t.uq[p][j], xs[j], magic, da, du);
      a = fmaf(bf_lo(gsw), da, fmaf(bf_hi(gsw), xs[j].xs, a));
      u = fmaf(bf_lo(usw), du, fmaf(bf_hi(usw), xs[j].xs, u));
    }
    a = seg_sum(a, m.lg);
    u = seg_sum(u, m.lg);
    const int r = row0 + p * m.rpp + m.rip;
    if (m.li == 0 && r < I) h_out[r] = valid ? silu_mul(a, u) : __builtin_nanf("");
  }
}

// ---------------------------------------------------------------------------
// top-K of E logits by one wave: K rounds of (wave maximum, lowest index that
// holds it), then the softmax weights of the selected experts
// ([openclawradar] "Pipeline performance": softmax + topK routing).
// Lane l holds experts e = 64 i + l, so each load is one coalesced row.  A
// selected (or absent) entry becomes NaN, which the maximum skips; a NaN
// logit is never selected.
// ---------------------------------------------------------------------------
constexpr int kTopkNpl = kMaxE / 64;

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  // every lane of each 16-lane row now holds its row's maximum
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// The logits of one token.  E <= 512: lane l holds experts 8l .. 8l+7 in
// v[0..7] (contiguous, for the lane-sort selection below); otherwise one
// register per 64 experts (expert 64 i + l in v[i]).
__device__ __forceinline__ void topk_load(const float *__restrict__ lg, int E,
                                          float (&v)[kTopkNpl]) {
  const int lane = lane_id();
  if (E <= 512) {  // wave-uniform
    const int e0 = lane * 8;
    if ((E & 7) == 0) {
      const float4 *q = reinterpret_cast<const float4 *>(lg + (e0 < E ? e0 : 0));
      const float4 a = q[0], b = q[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = lg[e0 + i < E ? e0 + i : 0];
    }
#pragma unroll
    for (int i = 8; i < kTopkNpl; ++i) v[i] = -INFINITY;
    return;
  }
#pragma unroll
  for (int i = 0; i < kTopkNpl; ++i) {
    const int e = i * 64 + lane;
    v[i] = __builtin_nanf("");
    if (i * 64 < E) {  // wave-uniform
      // canonical values let the maxima below skip their NaN quieting
      const float l = __builtin_canonicalizef(lg[e < E ? e : 0]);
      v[i] = e < E ? l : __builtin_nanf("");
    }
  }
}

// Selection on the loaded logits, of which the first NPL registers hold
// experts (the others are NaN).  Lane k < K comes back with the k-th selected
// expert (descending logit; -2 if fewer than k+1 logits are numbers) in e_out
// and its weight in w_out; the other lanes get -2 and NaN.
template <int NPL>
__device__ __forceinline__ void topk_select_n(float (&v)[kTopkNpl], int K, int renorm,
                                              int &e_out, float &w_out) {
  const int lane = lane_id();
  float my_l = __builtin_nanf("");
  int my_e = -2;
  float mx = __builtin_nanf("");
#pragma unroll 1
  for (int k = 0; k < K; ++k) {
    float m = v[0];
#pragma unroll
    for (int i = 1; i < NPL; ++i) m = fmaxf(m, v[i]);
    m = wave_max(m);
    // lowest expert index that holds the maximum
    int sel = -2;
#pragma unroll
    for (int i = NPL - 1; i >= 0; --i) {
      const uint64_t b = __ballot(v[i] == m);
      if (b) sel = i * 64 + __builtin_ctzll(b);
    }
    sel = wave_uniform(sel);
    const int si = sel >> 6, sl = sel & 63;  // sel < 0 matches no lane
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (i == si && lane == sl) v[i] = __builtin_nanf("");
    if (lane == k) {
      my_l = m;
      my_e = sel;
    }
    if (k == 0) mx = m;
  }
  const bool mine = lane < K && my_e >= 0;
  const float t = mine ? expf(my_l - mx) : 0.f;
  float z = t;
  if (!renorm) {
    // the unselected experts join the denominator
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (!__builtin_isnan(v[i])) z += expf(v[i] - mx);
  }
  const float den = seg_sum(z, 6);
  e_out = my_e;
  w_out = mine ? t / den : __builtin_nanf("");
}

// Order-preserving unsigned key of a logit: larger logit, larger key.  NaN
// maps to the key of -inf and -0 to that of +0, so that logits equal as
// floats get equal keys.
__device__ __forceinline__ uint32_t logit_key(float f) {
  f = __builtin_isnan(f) ? -INFINITY : f + 0.0f;
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_logit(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  // every lane of each 16-lane row now holds its row's maximum
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}

// E <= 512 (lane-contiguous layout of topk_load).  Each logit becomes the
// 64-bit word (key << 32) | (2^32 - 1 - expert): a larger word is a larger
// logit, or an equal logit with a lower expert.  Every lane sorts its 8 words
// with the 19-comparator, depth-6 network of moe_sortnet.h; each of the K
// rounds is then a wave maximum of the lanes' first keys, the lowest lane
// holding it (lanes own increasing expert ranges, so that is the lowest
// expert among equal logits) and a shift of that lane's list.
__device__ __forceinline__ void topk_select8(float (&v)[kTopkNpl], int E, int K, int renorm,
                                             int &e_out, float &w_out) {
  const int lane = lane_id();
  uint64_t c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = lane * 8 + i;
    c[i] = e < E ? ((uint64_t)logit_key(v[i]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e) : 0ull;
    v[i] = e < E ? key_logit(logit_key(v[i])) : -INFINITY;  // for the softmax denominator
  }
#define MOE_CX(i, j)                          \
  do {                                        \
    const bool sw_ = c[j] > c[i];             \
    const uint64_t t_ = sw_ ? c[j] : c[i];    \
    c[j] = sw_ ? c[i] : c[j];                 \
    c[i] = t_;                                \
  } while (0)
#pragma unroll
  for (int q = 0; q < kSort8Comparators; ++q) MOE_CX(kSort8Net[q][0], kSort8Net[q][1]);
#undef MOE_CX
  uint32_t my_k = 0;
  int my_e = -2;
  uint32_t k0 = 0;
#pragma unroll 1
  for (int k = 0; k < K; ++k) {
    const uint32_t m = wave_max_u32((uint32_t)(c[0] >> 32));
    const uint64_t b = __ballot((uint32_t)(c[0] >> 32) == m);
    const int src = __builtin_ctzll(b);  // b != 0: m is some lane's key
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)c[0], src);
    const uint32_t ex = 0xFFFFFFFFu - lo;
    const int sel = (m != 0 && ex < (uint32_t)E) ? (int)ex : -2;
    if (lane == src) {  // shift the winner's list
#pragma unroll
      for (int i = 0; i < 7; ++i) c[i] = c[i + 1];
      c[7] = 0ull;
    }
    if (lane == k) {
      my_k = m;
      my_e = sel;
    }
    if (k == 0) k0 = m;
  }
  const float mx = key_logit(k0);
  const bool mine = lane < K && my_e >= 0;
  const float t = mine ? expf(key_logit(my_k) - mx) : 0.f;
  float z = t;
  if (!renorm) {
    z = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) z += expf(v[i] - mx);
  }
  const float den = seg_sum(z, 6);
  e_out = my_e;
  w_out = mine ? t / den : __builtin_nanf("");
}

__device__ __forceinline__ void topk_select(float (&v)[kTopkNpl], int E, int K, int renorm,
                                            int &e_out, float &w_out) {
  static_assert(kTopkNpl == 16, "expert registers of the wide layout");
  if (E <= 512) topk_select8(v, E, K, renorm, e_out, w_out);
  else topk_select_n<16>(v, K, renorm, e_out, w_out);
}

// ---------------------------------------------------------------------------
// top-K by the four waves of a workgroup together (E <= 1024).  Wave w takes
// the experts [w R, (w + 1) R) with R = 64 NPL, lane l the NPL consecutive
// experts w R + NPL l + i (NPL = 2 for E <= 512, else 4).  Each wave finds its
// own top K with the keyed-word rounds of topk_select8 and leaves them in LDS
// with its softmax partial (its maximum and the sum of exp(l - maximum) over
// its experts); after the workgroup's barrier every wave merges the 4 K
// candidates itself.  The words carry the expert, so the merge orders equal
// logits by the lower expert as the one-wave selection does.
// ---------------------------------------------------------------------------
struct alignas(16) TopkShare {
  uint64_t cand[4][kMaxK];
  float pmax[4], psum[4];
};

__device__ __forceinline__ int topk_npl(int E) { return E <= 256 * 2 ? 2 : 4; }

template <int NPL>
__device__ __forceinline__ void topk_part_load(const float *__restrict__ lg, int E, int w,
                                               float (&v)[4]) {
  const int e0 = (w * 64 + lane_id()) * NPL;
  if ((E % NPL) == 0) {  // wave-uniform
    if constexpr (NPL == 2) {
      const float2 a = *reinterpret_cast<const float2 *>(lg + (e0 < E ? e0 : 0));
      v[0] = a.x; v[1] = a.y;
    } else {
      const float4 a = *reinterpret_cast<const float4 *>(lg + (e0 < E ? e0 : 0));
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NPL; ++i) v[i] = lg[e0 + i < E ? e0 + i : 0];
  }
}

template <int NPL>
__device__ __forceinline__ void topk_part_select(const float (&v)[4], int E, int K, int renorm,
                                                 int w, TopkShare &sh) {
  const int lane = lane_id();
  const int e0 = (w * 64 + lane) * NPL;
  uint64_t c[NPL];
  float vl[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = e0 + i;
    const uint32_t key = logit_key(v[i]);
    c[i] = e < E ? ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e) : 0ull;
    vl[i] = e < E ? key_logit(key) : -INFINITY;  // for the softmax partial
  }
#define MOE_CX(i, j)                          \
  do {                                        \
    const bool sw_ = c[j] > c[i];             \
    const uint64_t t_ = sw_ ? c[j] : c[i];    \
    c[j] = sw_ ? c[i] : c[j];                 \
    c[i] = t_;                                \
  } while (0)
  if constexpr (NPL == 2) {
    MOE_CX(0, 1);
  } else {
    MOE_CX(0, 1); MOE_CX(2, 3); MOE_CX(0, 2); MOE_CX(1, 3); MOE_CX(1, 2);
  }
#undef MOE_CX
  uint32_t k0 = 0;
#pragma unroll 1
  for (int k = 0; k < K; ++k) {
    const uint32_t m = wave_max_u32((uint32_t)(c[0] >> 32));
    const uint64_t b = __ballot((uint32_t)(c[0] >> 32) == m);
    const int src = __builtin_ctzll(b);  // b != 0: m is some lane's key
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)c[0], src);
    if (lane == 0) sh.cand[w][k] = ((uint64_t)m << 32) | lo;
    if (lane == src) {  // shift the winner's list
#pragma unroll
      for (int i = 0; i < NPL - 1; ++i) c[i] = c[i + 1];
      c[NPL - 1] = 0ull;
    }
    if (k == 0) k0 = m;
  }
  if (!renorm) {
    // a wave without experts, or whose logits are all -inf, adds nothing
    const float mx = k0 ? key_logit(k0) : -INFINITY;
    float z = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int i = 0; i < NPL; ++i) z += expf(vl[i] - mx);
    }
    z = seg_sum(z, 6);
    if (lane == 0) {
      sh.pmax[w] = mx;
      sh.psum[w] = z;
    }
  }
}

// After the barrier: lane k < K comes back with the k-th selected expert
// (descending logit, the lower expert first among equal ones; -2 if there is
// none) in e_out; key_out holds its key and top_key the largest key, for
// topk_merge_weight.
__device__ __forceinline__ void topk_merge(const TopkShare &sh, int E, int K, int &e_out,
                                           uint32_t &key_out, uint32_t &top_key) {
  const int lane = lane_id();
  const bool has = lane < 4 * K;
  const int j = has ? lane : 0;  // candidate r of wave q, for lane j = q K + r
  const uint64_t cw0 = sh.cand[j / K][j - (j / K) * K];
  const uint64_t cw = has ? cw0 : 0ull;
  uint32_t hi = (uint32_t)(cw >> 32), lo = (uint32_t)cw;
  int my_e = -2;
  uint32_t my_k = 0, k0 = 0;
#pragma unroll 1
  for (int k = 0; k < K; ++k) {
    const uint32_t m = wave_max_u32(hi);
    const uint32_t ml = wave_max_u32(hi == m ? lo : 0u);
    const uint64_t b = __ballot(hi == m && lo == ml);
    const int src = __builtin_ctzll(b);  // the words are distinct: one lane
    const uint32_t ex = 0xFFFFFFFFu - ml;
    const int sel = (m != 0 && ex < (uint32_t)E) ? (int)ex : -2;
    if (lane == src) hi = lo = 0u;
    if (lane == k) {
      my_k = m;
      my_e = sel;
    }
    if (k == 0) k0 = m;
  }
  e_out = my_e;
  key_out = my_k;
  top_key = k0;
}

// Entry k (wave-uniform, 0 <= k < K) of the same selection alone, for a wave
// that needs one expert: lane j < 4K counts the candidate words larger than
// its own (LDS broadcast reads), and the word with exactly k larger ones is
// the k-th largest.  Real candidates are distinct words; an absent one is 0,
// and zeros rank after every real word, so a rank that only zeros (or no
// word) hold gives -2, as in topk_merge.
__device__ __forceinline__ int topk_merge_one(const TopkShare &sh, int E, int K, int k) {
  const int lane = lane_id();
  const bool has = lane < 4 * K;
  const int j = has ? lane : 0;
  const int q = j / K;
  const uint64_t cw = sh.cand[q][j - q * K];
  // every word is read before any comparison (16-byte broadcast reads, all
  // in flight together); a word at r >= K is not a candidate and is masked
  int rank = 0;
  auto count = [&](auto nr) {
    constexpr int NR = decltype(nr)::value;
    uint64_t o[4][NR];
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int r = 0; r < NR; r += 2) {
        const uint4 u = *reinterpret_cast<const uint4 *>(&sh.cand[w][r]);
        o[w][r] = ((uint64_t)u.y << 32) | u.x;
        o[w][r + 1] = ((uint64_t)u.w << 32) | u.z;
      }
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int r = 0; r < NR; ++r) rank += (r < K && o[w][r] > cw) ? 1 : 0;
  };
  if (K <= 4) count(std::integral_constant<int, 4>{});
  else count(std::integral_constant<int, kMaxK>{});
  const uint64_t b = __ballot(has && rank == k);
  if (!b) return -2;
  const int src = __builtin_ctzll(b);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(cw >> 32), src);
  const uint32_t ex = 0xFFFFFFFFu - __builtin_amdgcn_readlane((uint32_t)cw, src);
  return (hi != 0 && ex < (uint32_t)E) ? (int)ex : -2;
}

// The softmax weight of lane k's selection (lanes k < K; NaN elsewhere):
// over the K selected logits (renorm), or over all E, from the waves' partials.
__device__ __forceinline__ float topk_merge_weight(const TopkShare &sh, int K, int renorm, int e,
                                                   uint32_t key, uint32_t top_key) {
  const int lane = lane_id();
  const float mx = key_logit(top_key);
  const bool mine = lane < K && e >= 0;
  const float t = mine ? expf(key_logit(key) - mx) : 0.f;
  float den;
  if (renorm) {
    den = seg_sum(t, 6);
  } else {
    den = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (sh.pmax[w] != -INFINITY) den += sh.psum[w] * expf(sh.pmax[w] - mx);
  }
  return mine ? t / den : __builtin_nanf("");
}

// lanes 0..K-1 write the selection
__device__ __forceinline__ void topk_store(int e, float w, int K, int32_t *idx, float *wout) {
  const int lane = lane_id();
  if (lane < K) {
    if (idx) idx[lane] = e;
    if (wout) wout[lane] = w;
  }
}

// ---------------------------------------------------------------------------
// routing accumulators of stack layers (kAccCopies copies per entry, fp64)
// ---------------------------------------------------------------------------
// fp64 sum of entry e's copies, in copy order
__device__ __forceinline__ double acc_entry(const double *acc, int E, int e) {
  const int st = acc_stride(E);
  double s = 0.0;
#pragma unroll
  for (int c = 0; c < kAccCopies; ++c) s += acc[(size_t)c * st + e];
  return s;
}

// the norm's reciprocal r = 1 / sqrt(mean(v^2) + 1e-6) from entry E + 1
__device__ __forceinline__ float acc_rnorm(const double *acc, int E, int H) {
  return (float)(1.0 / sqrt(acc_entry(acc, E, E + 1) / (double)H + 1e-6));
}

// the split selection's logits (topk_part_load's layout) from the
// accumulators: logit = r * dot
template <int NPL>
__device__ __forceinline__ void topk_part_load_acc(const double *acc, int E, int w, float r,
                                                   float (&v)[4]) {
  const int e0 = (w * 64 + lane_id()) * NPL;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = e0 + i;
    v[i] = (float)acc_entry(acc, E, e < E ? e : 0) * r;
  }
}

// dot of columns [c0, c0 + n) of a router / gate row (fp32 or bf16) with
// v[0..n) in LDS; n a multiple of 8
__device__ __forceinline__ float slice_dot(const void *row, int dtype, int c0, int n, const float *v) {
  float a = 0.f;
  if (dtype == 1) {
    const uint4 *w = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(row) + c0);
    for (int j = 0; j < n / 8; ++j) {
      const uint4 u = w[j];
      const float *x = v + 8 * j;
      a = fmaf(bf_lo(u.x), x[0], a); a = fmaf(bf_hi(u.x), x[1], a);
      a = fmaf(bf_lo(u.y), x[2], a); a = fmaf(bf_hi(u.y), x[3], a);
      a = fmaf(bf_lo(u.z), x[4], a); a = fmaf(bf_hi(u.z), x[5], a);
      a = fmaf(bf_lo(u.w), x[6], a); a = fmaf(bf_hi(u.w), x[7], a);
    }
  } else {
    const float4 *w = reinterpret_cast<const float4 *>(static_cast<const float *>(row) + c0);
    for (int j = 0; j < n / 4; ++j) {
      const float4 u = w[j];
      const float *x = v + 4 * j;
      a = fmaf(u.x, x[0], a); a = fmaf(u.y, x[1], a);
      a = fmaf(u.z, x[2], a); a = fmaf(u.w, x[3], a);
    }
  }
  return a;
}

// the same with the first 64 bytes of the slice already in registers
__device__ __forceinline__ float slice_dot_pre(const uint4 (&pre)[4], int dtype, int n, const float *v) {
  float a = 0.f;
  if (dtype == 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (8 * j < n) {
        const uint4 u = pre[j];
        const float *x = v + 8 * j;
        a = fmaf(bf_lo(u.x), x[0], a); a = fmaf(bf_hi(u.x), x[1], a);
        a = fmaf(bf_lo(u.y), x[2], a); a = fmaf(bf_hi(u.y), x[3], a);
        a = fmaf(bf_lo(u.z), x[4], a); a = fmaf(bf_hi(u.z), x[5], a);
        a = fmaf(bf_lo(u.w), x[6], a); a = fmaf(bf_hi(u.w), x[7], a);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (4 * j < n) {
        const uint4 u = pre[j];
        const float *x = v + 4 * j;
        a = fmaf(__uint_as_float(u.x), x[0], a); a = fmaf(__uint_as_float(u.y), x[1], a);
        a = fmaf(__uint_as_float(u.z), x[2], a); a = fmaf(__uint_as_float(u.w), x[3], a);
      }
    }
  }
  return a;
}

// whether the first 64 bytes hold a whole slice of n columns
__host__ __device__ __forceinline__ bool slice_fits_pre(int dtype, int n) {
  return n * (dtype == 1 ? 2 : 4) <= 64;
}

// request router row e's slice of n columns at column c0 (n * element size
// <= 64 bytes: slice_fits_pre); nothing past the slice is read
__device__ __forceinline__ void slice_prefetch(const void *router, int dtype, int H, int e, int c0,
                                               int n, uint4 (&pre)[4]) {
  const int esz = dtype == 1 ? 2 : 4;
  const uint4 *w = reinterpret_cast<const uint4 *>(static_cast<const uint8_t *>(router) +
                                                   ((size_t)e * H + c0) * esz);
#pragma unroll
  for (int j = 0; j < 4; ++j) pre[j] = 16 * j < n * esz ? w[j] : make_uint4(0u, 0u, 0u, 0u);
}

// the same slice from the column tiles of the router (moe_router_tile: tile t
// holds columns 8t..8t+7 of every expert, 8 * element size bytes each); c0 a
// multiple of 8.  Fills pre exactly as slice_prefetch does.
__device__ __forceinline__ void slice_prefetch_tiles(const void *tiles, int dtype, int E, int e, int c0,
                                                     int n, uint4 (&pre)[4]) {
  const uint4 *w = static_cast<const uint4 *>(tiles);
  const int t0 = c0 / 8;
  if (dtype == 1) {  // one 16-byte run per tile
#pragma unroll
    for (int j = 0; j < 4; ++j) pre[j] = 16 * j < n * 2 ? w[(size_t)(t0 + j) * E + e] : make_uint4(0u, 0u, 0u, 0u);
  } else {           // two 16-byte halves per tile
#pragma unroll
    for (int j = 0; j < 4; ++j)
      pre[j] = 16 * j < n * 4 ? w[((size_t)(t0 + j / 2) * E + e) * 2 + (j & 1)] : make_uint4(0u, 0u, 0u, 0u);
  }
}

// One workgroup's routing partials for its rows v[0..n) (LDS), columns
// [c0, c0 + n): entries e < E the router row dots, E the gate dot, E + 1 the
// sum of v^2, each added to copy `copy` of acc.  Thread t takes entries t,
// t + nthreads, ...; pre holds router row t's slice when use_pre, gpre the
// gate's slice when gate_pre (set only in the thread that takes entry E).
__device__ __forceinline__ void routing_partials(const void *router, int rdt, const void *gate,
                                                 int gdt, int E, int H, const float *v, int c0,
                                                 int n, double *acc, int copy, int nthreads,
                                                 const uint4 (&pre)[4], bool use_pre,
                                                 const uint4 (&gpre)[4], bool gate_pre) {
  const size_t resz = rdt == 1 ? 2 : 4;
  for (int e = threadIdx.x; e < E + 2; e += nthreads) {
    float part;
    if (e < E) {
      part = (use_pre && e == (int)threadIdx.x)
                 ? slice_dot_pre(pre, rdt, n, v)
                 : slice_dot(static_cast<const uint8_t *>(router) + (size_t)e * H * resz, rdt, c0, n, v);
    } else if (e == E) {
      part = gate_pre ? slice_dot_pre(gpre, gdt, n, v) : slice_dot(gate, gdt, c0, n, v);
    } else {
      part = 0.f;
      for (int j = 0; j < n; ++j) part = fmaf(v[j], v[j], part);
    }
    atomicAdd(acc + (size_t)copy * acc_stride(E) + e, (double)part);
  }
}

// ---------------------------------------------------------------------------
// K1: router rows, shared-gate row, shared expert gate/up, x staging
// ---------------------------------------------------------------------------
// dot of a router/gate row with x for token t; every lane reads 16-byte
// chunks lane, lane+64, ... of the row.  fp32 accumulation in two chains per
// lane, then a 6-step tree: reduction depth stays <= 40 for H = 4096, which
// bounds the fp32 error of a logit well below the top-K gap.
// the first 512 16-byte chunks of a row (all of a bf16 row up to 4096
// columns), loaded ahead of the activations they meet
struct RowPre {
  uint4 w[8];
};

__device__ __forceinline__ RowPre row_prefetch(const void *row, int dtype, int H) {
  RowPre r;
  const int U = dtype == 1 ? H / 8 : H / 4;
  const uint4 *W = static_cast<const uint4 *>(row);
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const int c = jj * 64 + lane_id();
    r.w[jj] = W[c < U ? c : 0];
  }
  return r;
}

template <int XS>
__device__ __forceinline__ float row_dot(const void *row, int dtype, int H, const void *x,
                                         const float *xl, int t, const RowPre &pre = RowPre{},
                                         bool use_pre = false) {
  const int lane = lane_id();
  float acc0 = 0.f, acc1 = 0.f;
  if (dtype == 1) {  // bf16 row: chunk c = columns 8c .. 8c+7
    const uint4 *W = static_cast<const uint4 *>(row);
    const int U = H / 8;
    for (int j0 = 0; j0 < U; j0 += 64 * 8) {
      uint4 wv[8];
      float4 xa[8], xb[8];
      uint4 xh[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int c = j0 + jj * 64 + lane;
        const int cc = c < U ? c : 0;
        wv[jj] = (use_pre && j0 == 0) ? pre.w[jj] : W[cc];
        if constexpr (XS == XS_BF16) {
          xh[jj] = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + (size_t)t * H)[cc];
        } else {
          const float *xf = (XS == XS_F32) ? static_cast<const float *>(x) + (size_t)t * H : xl;
          xa[jj] = reinterpret_cast<const float4 *>(xf)[2 * cc];
          xb[jj] = reinterpret_cast<const float4 *>(xf)[2 * cc + 1];
        }
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const bool in = j0 + jj * 64 + lane < U;
        const uint4 w = in ? wv[jj] : make_uint4(0, 0, 0, 0);
        if constexpr (XS == XS_BF16) {
          acc0 = dot2bf(w.x, xh[jj].x, acc0);
          acc1 = dot2bf(w.y, xh[jj].y, acc1);
          acc0 = dot2bf(w.z, xh[jj].z, acc0);
          acc1 = dot2bf(w.w, xh[jj].w, acc1);
        } else {
          const float4 a = xa[jj], b = xb[jj];
          acc0 = fmaf(bf_lo(w.x), a.x, acc0); acc1 = fmaf(bf_hi(w.x), a.y, acc1);
          acc0 = fmaf(bf_lo(w.y), a.z, acc0); acc1 = fmaf(bf_hi(w.y), a.w, acc1);
          acc0 = fmaf(bf_lo(w.z), b.x, acc0); acc1 = fmaf(bf_hi(w.z), b.y, acc1);
          acc0 = fmaf(bf_lo(w.w), b.z, acc0); acc1 = fmaf(bf_hi(w.w), b.w, acc1);
        }
      }
    }
  } else {  // fp32 row: chunk c = columns 4c .. 4c+3
    const float4 *W = static_cast<const float4 *>(row);
    const int U = H / 4;
    for (int j0 = 0; j0 < U; j0 += 64 * 8) {
      float4 wv[8], xv[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int c = j0 + jj * 64 + lane;
        const int cc = c < U ? c : 0;
        if (use_pre && j0 == 0) {
          const uint4 u = pre.w[jj];
          wv[jj] = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                               __uint_as_float(u.w));
        } else {
          wv[jj] = W[cc];
        }
        if constexpr (XS == XS_BF16) {
          const uint2 u = reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(x) + (size_t)t * H)[cc];
          xv[jj] = make_float4(bf_lo(u.x), bf_hi(u.x), bf_lo(u.y), bf_hi(u.y));
        } else {
          const float *xf = (XS == XS_F32) ? static_cast<const float *>(x) + (size_t)t * H : xl;
          xv[jj] = reinterpret_cast<const float4 *>(xf)[cc];
        }
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const bool in = j0 + jj * 64 + lane < U;
        const float4 w = in ? wv[jj] : make_float4(0.f, 0.f, 0.f, 0.f);
        acc0 = fmaf(w.x, xv[jj].x, acc0); acc1 = fmaf(w.y, xv[jj].y, acc1);
        acc0 = fmaf(w.z, xv[jj].z, acc0); acc1 = fmaf(w.w, xv[jj].w, acc1);
      }
    }
  }
  return seg_sum(acc0 + acc1, 6);
}

// x = (h + u) / sqrt(mean((h + u)^2) + 1e-6) into LDS, two passes
// ([openclawradar] "Metal compute shaders": RMS normalisation in two passes)
// x = RMSNorm(h + u) into LDS (every workgroup), h + u and x also to global
// memory from workgroup 0.  Each thread takes 4 consecutive columns per
// step; all loads are issued before the first use.
__device__ __forceinline__ void norm_prologue(const HeadParams &p, float *xl) {
  __shared__ float red[kBlock / 64];
  constexpr int kSteps = kMaxDim / (4 * kBlock);
  const int H = p.H;
  float4 hv[kSteps];
  uint2 uv[kSteps];
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int c = (i * kBlock + threadIdx.x) * 4;
    const int cc = c < H ? c : 0;
    hv[i] = *reinterpret_cast<const float4 *>(p.h_in + cc);
    uv[i] = p.upd ? *reinterpret_cast<const uint2 *>(p.upd + cc) : make_uint2(0u, 0u);
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int c = (i * kBlock + threadIdx.x) * 4;
    if (c < H) {
      float4 v = hv[i];
      v.x += bf_lo(uv[i].x);
      v.y += bf_hi(uv[i].x);
      v.z += bf_lo(uv[i].y);
      v.w += bf_hi(uv[i].y);
      hv[i] = v;
      ss = fmaf(v.x, v.x, ss);
      ss = fmaf(v.y, v.y, ss);
      ss = fmaf(v.z, v.z, ss);
      ss = fmaf(v.w, v.w, ss);
    }
  }
  ss = seg_sum(ss, 6);
  if (lane_id() == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < kBlock / 64; ++i) tot += red[i];
  const float rinv = 1.0f / sqrtf(tot / (float)H + 1e-6f);
  const bool w0 = blockIdx.x == 0;
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int c = (i * kBlock + threadIdx.x) * 4;
    if (c < H) {
      const float4 v = hv[i];
      const float4 xv = make_float4(v.x * rinv, v.y * rinv, v.z * rinv, v.w * rinv);
      *reinterpret_cast<float4 *>(xl + c) = xv;
      if (w0) {
        if (p.hres_out) *reinterpret_cast<float4 *>(p.hres_out + c) = v;
        if (p.x_out) *reinterpret_cast<float4 *>(p.x_out + c) = xv;
      }
    }
  }
  __syncthreads();
}

// The same normalisation for workgroups that only take dot products with x:
// x = v r with v = h + u and the scalar r = 1 / sqrt(mean(v^2) + eps), so a
// row's dot with x is r times its dot with v.  v goes to LDS in the pass that
// sums its squares, and one barrier serves both; workgroup 0 still writes the
// normalised x (and v) for the next kernels.  Returns r.
__device__ __forceinline__ float norm_prologue_scaled(const HeadParams &p, float *vl) {
  __shared__ float red[kBlock / 64];
  constexpr int kSteps = kMaxDim / (4 * kBlock);
  const int H = p.H;
  float4 hv[kSteps];
  uint2 uv[kSteps];
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int c = (i * kBlock + threadIdx.x) * 4;
    const int cc = c < H ? c : 0;
    hv[i] = *reinterpret_cast<const float4 *>(p.h_in + cc);
    uv[i] = p.upd ? *reinterpret_cast<const uint2 *>(p.upd + cc) : make_uint2(0u, 0u);
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int c = (i * kBlock + threadIdx.x) * 4;
    if (c < H) {
      float4 v = hv[i];
      v.x += bf_lo(uv[i].x);
      v.y += bf_hi(uv[i].x);
      v.z += bf_lo(uv[i].y);
      v.w += bf_hi(uv[i].y);
      hv[i] = v;
      ss = fmaf(v.x, v.x, ss);
      ss = fmaf(v.y, v.y, ss);
      ss = fmaf(v.z, v.z, ss);
      ss = fmaf(v.w, v.w, ss);
      *reinterpret_cast<float4 *>(vl + c) = v;
    }
  }
  ss = seg_sum(ss, 6);
  if (lane_id() == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < kBlock / 64; ++i) tot += red[i];
  const float rinv = 1.0f / sqrtf(tot / (float)H + 1e-6f);
  if (blockIdx.x == 0) {
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      const int c = (i * kBlock + threadIdx.x) * 4;
      if (c < H) {
        const float4 v = hv[i];
        if (p.hres_out) *reinterpret_cast<float4 *>(p.hres_out + c) = v;
        if (p.x_out)
          *reinterpret_cast<float4 *>(p.x_out + c) = make_float4(v.x * rinv, v.y * rinv, v.z * rinv, v.w * rinv);
      }
    }
  }
  return rinv;
}

// one wave stages bf16 x for every chunk of a row at BITS and stores it
template <int BITS>
__device__ __forceinline__ void write_xstage(const void *x, int H, uint32_t *pairs, float *sums) {
  constexpr int NP = ChunkGeom<BITS>::kPairs;
  const int cpr = H / ChunkGeom<BITS>::kCols;
  for (int c = lane_id(); c < cpr; c += 64) {
    const XStage<BITS, false> s = make_stage<BITS, XS_BF16>(x, nullptr, c);
    uint4 *pp = reinterpret_cast<uint4 *>(pairs + (size_t)c * NP);
#pragma unroll
    for (int i = 0; i < NP / 4; ++i)
      pp[i] = make_uint4(s.p[4 * i], s.p[4 * i + 1], s.p[4 * i + 2], s.p[4 * i + 3]);
    reinterpret_cast<float2 *>(sums)[c] = make_float2(s.off, s.xs);
  }
}

// ---------------------------------------------------------------------------
// K3: down projection
// ---------------------------------------------------------------------------
template <int BITS, int NCH, int NPASS>
struct DnTile {
  uint4 q[NPASS][NCH];
  uint32_t sb[NPASS][NCH];
};

template <int BITS, int NCH, int NPASS>
__device__ __forceinline__ void down_load(DnTile<BITS, NCH, NPASS> &t, const uint8_t *rec,
                                          const RecOffsets &off, int H, const RowMap &m,
                                          int row0) {
  const uint32_t *dc = reinterpret_cast<const uint32_t *>(rec + off.down_codes);
  const uint32_t *ds = reinterpret_cast<const uint32_t *>(rec + off.down_sb);
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int r = row0 + p * m.rpp + m.rip;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = m.li + (j << m.lg);
      const bool in = r < H && c < m.cpr;
      const int rr = in ? r : 0, cc = in ? c : 0;
      t.q[p][j] = *reinterpret_cast<const uint4 *>(dc + (size_t)rr * m.wpr + (size_t)cc * 4);
      t.sb[p][j] = ds[(size_t)rr * m.gpr + chunk_group<BITS>(cc)];
    }
  }
}

// a 64-bit pointer the wave holds in every lane, made wave-uniform
__device__ __forceinline__ uint64_t wave_uniform_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// weighted partial sums of one expert into acc[p]; the passes are taken in
// pairs so that two rows form independent accumulation chains
template <int BITS, int NCH, int NPASS>
__device__ __forceinline__ void down_accumulate_staged(const XStage<BITS, true> (&xs)[NCH],
                                                       const RowMap &m, int H, int row0, bool valid,
                                                       float wgt, const DnTile<BITS, NCH, NPASS> &t,
                                                       float (&acc)[NPASS]) {
#pragma unroll
  for (int p = 0; p < NPASS; p += 2) {
    constexpr int kLast = NPASS - 1;
    const int p1 = p + 1 <= kLast ? p + 1 : p;
    float part0 = 0.f, part1 = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const uint32_t s0 = in_tile(m, H, row0, p, j) ? t.sb[p][j] : 0u;
      const uint32_t s1 = in_tile(m, H, row0, p1, j) ? t.sb[p1][j] : 0u;
      float d0, d1;
      if (p1 != p) chunk_dot_f32<BITS, true>(t.q[p][j], t.q[p1][j], xs[j], d0, d1);
      else chunk_dot_f32<BITS, false>(t.q[p][j], t.q[p][j], xs[j], d0, d1);
      part0 = fmaf(bf_lo(s0), d0, fmaf(bf_hi(s0), xs[j].xs, part0));
      part1 = fmaf(bf_lo(s1), d1, fmaf(bf_hi(s1), xs[j].xs, part1));
    }
    acc[p] = valid ? fmaf(wgt, part0, acc[p]) : __builtin_nanf("");
    if (p1 != p) acc[p1] = valid ? fmaf(wgt, part1, acc[p1]) : __builtin_nanf("");
  }
}

// The same sums with the input staged one code chunk at a time (each pass's
// partial still takes the chunks in ascending order, so the result is bit for
// bit that of down_accumulate_staged): one chunk's columns are live at once
// instead of NCH of them, which keeps rows of several chunks per lane (long
// input dimensions) within the registers of four waves per SIMD.
template <int BITS, int NCH, int NPASS, int XS>
__device__ __forceinline__ void down_accumulate(const float *hin, const RowMap &m, int H,
                                                int row0, bool valid, float wgt,
                                                const DnTile<BITS, NCH, NPASS> &t,
                                                float (&acc)[NPASS]) {
  float part[NPASS];
#pragma unroll
  for (int p = 0; p < NPASS; ++p) part[p] = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = m.li + (j << m.lg);
    const XStage<BITS, true> xs = make_stage<BITS, XS>(hin, hin, c < m.cpr ? c : 0);
#pragma unroll
    for (int p = 0; p < NPASS; p += 2) {
      constexpr int kLast = NPASS - 1;
      const int p1 = p + 1 <= kLast ? p + 1 : p;
      const uint32_t s0 = in_tile(m, H, row0, p, j) ? t.sb[p][j] : 0u;
      const uint32_t s1 = in_tile(m, H, row0, p1, j) ? t.sb[p1][j] : 0u;
      float d0, d1;
      if (p1 != p) chunk_dot_f32<BITS, true>(t.q[p][j], t.q[p1][j], xs, d0, d1);
      else chunk_dot_f32<BITS, false>(t.q[p][j], t.q[p][j], xs, d0, d1);
      part[p] = fmaf(bf_lo(s0), d0, fmaf(bf_hi(s0), xs.xs, part[p]));
      if (p1 != p) part[p1] = fmaf(bf_lo(s1), d1, fmaf(bf_hi(s1), xs.xs, part[p1]));
    }
  }
#pragma unroll
  for (int p = 0; p < NPASS; ++p) acc[p] = valid ? fmaf(wgt, part[p], acc[p]) : __builtin_nanf("");
}

// ---------------------------------------------------------------------------
// host-side tile geometry (code chunks per lane, rows per pass of a wave)
// ---------------------------------------------------------------------------
inline int nch_for(int cols, int bits) {
  const int cpr = cols * bits / 128;
  const int lpr = cpr >= 64 ? 64 : (1 << ceil_log2(cpr));
  const int nch = (cpr + lpr - 1) / lpr;
  return nch <= 1 ? 1 : (nch <= 2 ? 2 : 4);
}
inline int rpp_for(int cols, int bits) {
  const int cpr = cols * bits / 128;
  int lg = ceil_log2(cpr);
  if (lg > 6) lg = 6;
  return 64 >> lg;
}
// rows of two code chunks per lane take at most two passes, of four one
inline int clamp_pass(int nch, int npass) {
  return nch >= 4 ? 1 : (nch >= 2 && npass > 2 ? 2 : npass);
}

}  // namespace moe_impl
