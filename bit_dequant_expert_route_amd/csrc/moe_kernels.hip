// moe_kernels.hip -- gfx950 kernels of the MoE expert hot path.
//
// Pages (cited by site and section):
//   [openclawradar] openclawradar.com (ja), "Flash-MoE: running the 397B
//       parameter Qwen model on a MacBook Pro in pure C/Metal"
//   [a2a-fr] a2a-mcp.org (fr), "What is Flash-MoE? Running 397B-parameter AI
//       models on a laptop"
//   [sardonic] education.sardonicrepulsion.com (sk), "Flash-MoE: how to run a
//       397-billion-parameter AI model on an ordinary notebook"
//
// The pages' dequant matvec computes sum_c (q*scale + bias) * x_c and rewrites
// it as fma(q, scale*x, bias*x) ([openclawradar] "FMA-optimized dequant
// kernel"; [sardonic] "FMA-optimised dequantisation kernel" gives
// fma(q*x, scale, bias*x)).  All are regroupings of one sum.  Here the sum is
// regrouped per 64-column group g (one scale s_g and bias b_g):
//     y = sum_g s_g * (sum_{c in g} q_c x_c) + b_g * (sum_{c in g} x_c)
// where the integer-weighted inner sums carry exact products: on the packed
// bf16 dot instruction (v_dot2_f32_bf16) when x is bf16, with codes made into
// bf16 numbers by OR-ing them into a mantissa; in fp32 FMAs after the byte
// converts when x is fp32.  x is staged once per lane (a lane always sees the
// same input columns) and the bias term needs only the chunk sums of x.
//
// Memory mapping: a wave reads whole quantised rows with 128-bit loads, lane l
// taking 16-byte chunks l, l+64, ... of a row (rows shorter than 64 chunks are
// packed several to a wave), so every load instruction covers one contiguous
// run of up to 1 KiB.  Rows are reduced with DPP / lane shuffles.
#include "moe_internal.h"

#include <math.h>
#include <stdint.h>

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
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
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

// hide a value's provenance so that the byte-select converts are formed
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// sum_c q_c * x_c over one 16-byte code chunk
template <int BITS>
__device__ __forceinline__ float chunk_dot(const uint4 &q, const XStage<BITS, false> &s,
                                           uint32_t kMagic16) {
  float acc = -s.off;
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t a = w[t] << 3, b = w[t] >> 1, c = w[t] >> 5, d = w[t] >> 9;
    if constexpr (BITS == 4) {
      acc = dot2bf((a & 0x00780078u) | kMagic16, s.p[4 * t + 0], acc);
      acc = dot2bf((b & 0x00780078u) | kMagic16, s.p[4 * t + 1], acc);
      acc = dot2bf((c & 0x00780078u) | kMagic16, s.p[4 * t + 2], acc);
      acc = dot2bf((d & 0x00780078u) | kMagic16, s.p[4 * t + 3], acc);
    } else {
      acc = dot2bf((a & 0x00180018u) | kMagic16, s.p[8 * t + 0], acc);
      acc = dot2bf((a & 0x00600060u) | kMagic16, s.p[8 * t + 1], acc);
      acc = dot2bf((b & 0x00180018u) | kMagic16, s.p[8 * t + 2], acc);
      acc = dot2bf((b & 0x00600060u) | kMagic16, s.p[8 * t + 3], acc);
      acc = dot2bf((c & 0x00180018u) | kMagic16, s.p[8 * t + 4], acc);
      acc = dot2bf((c & 0x00600060u) | kMagic16, s.p[8 * t + 5], acc);
      acc = dot2bf((d & 0x00180018u) | kMagic16, s.p[8 * t + 6], acc);
      acc = dot2bf((d & 0x00600060u) | kMagic16, s.p[8 * t + 7], acc);
    }
  }
  return acc;
}

template <int BITS>
__device__ __forceinline__ float chunk_dot(const uint4 &q, const XStage<BITS, true> &s) {
  float acc = 0.f;
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if constexpr (BITS == 4) {
      // bytes of lo: nibbles 0,2,4,6; bytes of hi: nibbles 1,3,5,7
      const uint32_t lo = opaque(w[t] & 0x0F0F0F0Fu);
      const uint32_t hi = opaque((w[t] >> 4) & 0x0F0F0F0Fu);
      const float *x = s.v + 8 * t;
      acc = fmaf((float)(lo & 0xFFu), x[0], acc);
      acc = fmaf((float)(hi & 0xFFu), x[1], acc);
      acc = fmaf((float)((lo >> 8) & 0xFFu), x[2], acc);
      acc = fmaf((float)((hi >> 8) & 0xFFu), x[3], acc);
      acc = fmaf((float)((lo >> 16) & 0xFFu), x[4], acc);
      acc = fmaf((float)((hi >> 16) & 0xFFu), x[5], acc);
      acc = fmaf((float)(lo >> 24), x[6], acc);
      acc = fmaf((float)(hi >> 24), x[7], acc);
    } else {
      // byte b of f_k is field 4b + k
      const uint32_t f0 = opaque(w[t] & 0x03030303u);
      const uint32_t f1 = opaque((w[t] >> 2) & 0x03030303u);
      const uint32_t f2 = opaque((w[t] >> 4) & 0x03030303u);
      const uint32_t f3 = opaque((w[t] >> 6) & 0x03030303u);
      const float *x = s.v + 16 * t;
      const uint32_t f[4] = {f0, f1, f2, f3};
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t byte = bb == 3 ? (f[k] >> 24) : ((f[k] >> (8 * bb)) & 0xFFu);
          acc = fmaf((float)byte, x[4 * bb + k], acc);
        }
      }
    }
  }
  return acc;
}

template <int BITS>
__device__ __forceinline__ float chunk_dot_any(const uint4 &q, const XStage<BITS, false> &s,
                                               uint32_t magic) {
  return chunk_dot<BITS>(q, s, magic);
}
template <int BITS>
__device__ __forceinline__ float chunk_dot_any(const uint4 &q, const XStage<BITS, true> &s,
                                               uint32_t) {
  return chunk_dot<BITS>(q, s);
}

// load the x values of one chunk (columns col0 .. col0 + kCols - 1) as fp32
template <int BITS, int XS>
__device__ __forceinline__ void load_x_chunk(const void *x, const float *xl, int col0,
                                             float (&v)[ChunkGeom<BITS>::kCols]) {
  constexpr int NC = ChunkGeom<BITS>::kCols;
  if constexpr (XS == XS_BF16) {
    const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + col0);
#pragma unroll
    for (int i = 0; i < NC / 8; ++i) {
      const uint4 u = p[i];
      v[8 * i + 0] = bf_lo(u.x); v[8 * i + 1] = bf_hi(u.x);
      v[8 * i + 2] = bf_lo(u.y); v[8 * i + 3] = bf_hi(u.y);
      v[8 * i + 4] = bf_lo(u.z); v[8 * i + 5] = bf_hi(u.z);
      v[8 * i + 6] = bf_lo(u.w); v[8 * i + 7] = bf_hi(u.w);
    }
  } else if constexpr (XS == XS_F32) {
    const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(x) + col0);
#pragma unroll
    for (int i = 0; i < NC / 4; ++i) {
      const float4 u = p[i];
      v[4 * i + 0] = u.x; v[4 * i + 1] = u.y; v[4 * i + 2] = u.z; v[4 * i + 3] = u.w;
    }
  } else {
    const float4 *p = reinterpret_cast<const float4 *>(xl + col0);
#pragma unroll
    for (int i = 0; i < NC / 4; ++i) {
      const float4 u = p[i];
      v[4 * i + 0] = u.x; v[4 * i + 1] = u.y; v[4 * i + 2] = u.z; v[4 * i + 3] = u.w;
    }
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
// gate/up + SwiGLU for rows [row0, row0 + NPASS*rpp) of one expert
// ([openclawradar] "Metal compute shaders": fused SwiGLU; h = silu(a) * u)
// ---------------------------------------------------------------------------
template <int BITS, int NCH, int NPASS, int XS>
__device__ __forceinline__ void gateup_wave(const uint8_t *rec, const RecOffsets &off,
                                            int H, int I, int row0, bool valid,
                                            const void *x, const float *xl, float *h_out) {
  constexpr bool XF32 = (XS != XS_BF16);
  const RowMap m = row_map<BITS>(H);
  const uint32_t *gc = reinterpret_cast<const uint32_t *>(rec + off.gate_codes);
  const uint32_t *uc = reinterpret_cast<const uint32_t *>(rec + off.up_codes);
  const uint32_t *gs = reinterpret_cast<const uint32_t *>(rec + off.gate_sb);
  const uint32_t *us = reinterpret_cast<const uint32_t *>(rec + off.up_sb);

  uint4 gq[NPASS][NCH], uq[NPASS][NCH];
  uint32_t gsw[NPASS][NCH], usw[NPASS][NCH];
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int r = row0 + p * m.rpp + m.rip;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = m.li + (j << m.lg);
      if (valid && r < I && c < m.cpr) {
        const size_t wo = (size_t)r * m.wpr + (size_t)c * 4;
        gq[p][j] = *reinterpret_cast<const uint4 *>(gc + wo);
        uq[p][j] = *reinterpret_cast<const uint4 *>(uc + wo);
        const size_t so = (size_t)r * m.gpr + chunk_group<BITS>(c);
        gsw[p][j] = gs[so];
        usw[p][j] = us[so];
      } else {
        gq[p][j] = make_uint4(0, 0, 0, 0);
        uq[p][j] = make_uint4(0, 0, 0, 0);
        gsw[p][j] = 0;
        usw[p][j] = 0;
      }
    }
  }

  XStage<BITS, XF32> xs[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = m.li + (j << m.lg);
    if (c < m.cpr) {
      float v[ChunkGeom<BITS>::kCols];
      load_x_chunk<BITS, XS>(x, xl, c * ChunkGeom<BITS>::kCols, v);
      stage_chunk<BITS>(v, xs[j]);
    }
  }

  // the magic constant lives in a VGPR so that mask-and-or is one v_and_or_b32
  // (gfx9 VOP3 reads at most one scalar or literal operand)
  const uint32_t magic = opaque(kMagic16);
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    float a = 0.f, u = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = m.li + (j << m.lg);
      if (c < m.cpr) {
        const float da = chunk_dot_any<BITS>(gq[p][j], xs[j], magic);
        const float du = chunk_dot_any<BITS>(uq[p][j], xs[j], magic);
        a = fmaf(bf_lo(gsw[p][j]), da, fmaf(bf_hi(gsw[p][j]), xs[j].xs, a));
        u = fmaf(bf_lo(usw[p][j]), du, fmaf(bf_hi(usw[p][j]), xs[j].xs, u));
      }
    }
    a = seg_sum(a, m.lg);
    u = seg_sum(u, m.lg);
    const int r = row0 + p * m.rpp + m.rip;
    if (m.li == 0 && r < I) h_out[r] = valid ? silu_mul(a, u) : __builtin_nanf("");
  }
}

// ---------------------------------------------------------------------------
// top-K of E logits by one wave: K selection rounds of a wave arg-max, ties to
// the lower index; then softmax weights of the selected experts
// ([openclawradar] "Pipeline performance": softmax + topK routing)
// ---------------------------------------------------------------------------
struct TopK {
  int idx[kMaxK];
  float w[kMaxK];
};

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ TopK wave_topk(const float *__restrict__ lg, int E, int K, int renorm) {
  const int lane = lane_id();
  constexpr int NV = kMaxE / 64;
  float v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? lg[e] : -INFINITY;
  }
  uint32_t taken = 0;
  TopK r;
  float lk[kMaxK];
#pragma unroll
  for (int k = 0; k < kMaxK; ++k) {
    r.idx[k] = -2;
    r.w[k] = 0.f;
    lk[k] = -INFINITY;
    if (k < K) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int e = lane + 64 * i;
        if (e < E && !((taken >> i) & 1u) && better(v[i], e, bv, bi)) {
          bv = v[i];
          bi = e;
        }
      }
#pragma unroll
      for (int msk = 32; msk >= 1; msk >>= 1) {
        const float ov = __shfl_xor(bv, msk, 64);
        const int oi = __shfl_xor(bi, msk, 64);
        if (better(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if (bi != 0x7fffffff && (bi & 63) == lane) taken |= 1u << (bi >> 6);
      r.idx[k] = bi == 0x7fffffff ? -2 : bi;
      lk[k] = bv;
    }
  }
  const float mx = lk[0];
  float z = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i;
    if (e < E) z += expf(v[i] - mx);
  }
  z = seg_sum(z, 6);
  float zk = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxK; ++k)
    if (k < K) zk += expf(lk[k] - mx);
  const float den = renorm ? zk : z;
#pragma unroll
  for (int k = 0; k < kMaxK; ++k) {
    if (k < K) r.w[k] = r.idx[k] < 0 ? __builtin_nanf("") : expf(lk[k] - mx) / den;
  }
  return r;
}

__device__ __forceinline__ int pick_idx(const TopK &t, int k) {
  int v = -2;
#pragma unroll
  for (int i = 0; i < kMaxK; ++i)
    if (i == k) v = t.idx[i];
  return v;
}

__device__ __forceinline__ void write_topk(const TopK &t, int K, int32_t *idx, float *w) {
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < kMaxK; ++i) {
    if (i < K && lane == i) {
      if (idx) idx[i] = t.idx[i];
      if (w) w[i] = t.w[i];
    }
  }
}

// ---------------------------------------------------------------------------
// K1: router rows, shared-gate row, shared expert gate/up
// ---------------------------------------------------------------------------
// dot of a router/gate row with x for token t; every lane reads 16-byte
// chunks lane, lane+64, ... of the row.  fp32 accumulation per lane, then a
// 6-step tree: reduction depth stays <= 70 for H = 4096, which bounds the
// fp32 error of a logit well below the top-K gap.
template <int XS>
__device__ __forceinline__ float row_dot(const void *row, int dtype, int H, const void *x,
                                         const float *xl, int t) {
  const int lane = lane_id();
  float acc = 0.f;
  if (dtype == 1) {  // bf16 row
    const uint4 *W = static_cast<const uint4 *>(row);
    const int U = H / 8;
    for (int j0 = 0; j0 < U; j0 += 64 * 8) {
      uint4 wv[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int c = j0 + jj * 64 + lane;
        wv[jj] = c < U ? W[c] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int c = j0 + jj * 64 + lane;
        if (c < U) {
          const uint32_t w4[4] = {wv[jj].x, wv[jj].y, wv[jj].z, wv[jj].w};
          if constexpr (XS == XS_BF16) {
            const uint4 xv = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + (size_t)t * H)[c];
            acc = dot2bf(w4[0], xv.x, acc);
            acc = dot2bf(w4[1], xv.y, acc);
            acc = dot2bf(w4[2], xv.z, acc);
            acc = dot2bf(w4[3], xv.w, acc);
          } else {
            const float *xf = (XS == XS_F32) ? static_cast<const float *>(x) + (size_t)t * H : xl;
            const float4 a = reinterpret_cast<const float4 *>(xf)[2 * c];
            const float4 b = reinterpret_cast<const float4 *>(xf)[2 * c + 1];
            acc = fmaf(bf_lo(w4[0]), a.x, acc); acc = fmaf(bf_hi(w4[0]), a.y, acc);
            acc = fmaf(bf_lo(w4[1]), a.z, acc); acc = fmaf(bf_hi(w4[1]), a.w, acc);
            acc = fmaf(bf_lo(w4[2]), b.x, acc); acc = fmaf(bf_hi(w4[2]), b.y, acc);
            acc = fmaf(bf_lo(w4[3]), b.z, acc); acc = fmaf(bf_hi(w4[3]), b.w, acc);
          }
        }
      }
    }
  } else {  // fp32 row
    const float4 *W = static_cast<const float4 *>(row);
    const int U = H / 4;
    for (int j0 = 0; j0 < U; j0 += 64 * 8) {
      float4 wv[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int c = j0 + jj * 64 + lane;
        wv[jj] = c < U ? W[c] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int c = j0 + jj * 64 + lane;
        if (c < U) {
          float4 xv;
          if constexpr (XS == XS_BF16) {
            const uint2 u = reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(x) + (size_t)t * H)[c];
            xv = make_float4(bf_lo(u.x), bf_hi(u.x), bf_lo(u.y), bf_hi(u.y));
          } else {
            const float *xf = (XS == XS_F32) ? static_cast<const float *>(x) + (size_t)t * H : xl;
            xv = reinterpret_cast<const float4 *>(xf)[c];
          }
          acc = fmaf(wv[jj].x, xv.x, acc); acc = fmaf(wv[jj].y, xv.y, acc);
          acc = fmaf(wv[jj].z, xv.z, acc); acc = fmaf(wv[jj].w, xv.w, acc);
        }
      }
    }
  }
  return seg_sum(acc, 6);
}

// x = (h + u) / sqrt(mean((h + u)^2) + 1e-6) into LDS, two passes
// ([openclawradar] "Metal compute shaders": RMS normalisation in two passes)
__device__ __forceinline__ void norm_prologue(const HeadParams &p, float *xl) {
  __shared__ float red[kBlock / 64];
  const int H = p.H;
  float ss = 0.f;
  for (int c = threadIdx.x; c < H; c += kBlock) {
    float v = p.h_in[c];
    if (p.upd) v += __uint_as_float(static_cast<uint32_t>(p.upd[c]) << 16);
    xl[c] = v;
    ss = fmaf(v, v, ss);
  }
  ss = seg_sum(ss, 6);
  if (lane_id() == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < kBlock / 64; ++i) tot += red[i];
  const float rinv = 1.0f / sqrtf(tot / (float)H + 1e-6f);
  const bool w0 = blockIdx.x == 0;
  for (int c = threadIdx.x; c < H; c += kBlock) {
    const float v = xl[c];
    const float xv = v * rinv;
    xl[c] = xv;
    if (w0) {
      if (p.hres_out) p.hres_out[c] = v;
      if (p.x_out) p.x_out[c] = xv;
    }
  }
  __syncthreads();
}

template <int XS, int BITS_S, int NCH_S, int NPASS_S>
__global__ __launch_bounds__(kBlock) void k_head(HeadParams p) {
  extern __shared__ float xl[];
  if constexpr (XS == XS_NORM) norm_prologue(p, xl);
  const int wv = wave_uniform(threadIdx.x >> 6);
  const int blk = wave_uniform(blockIdx.x);
  if (blk < p.n_router_blocks) {
    const int unit = blk * (kBlock / 64) + wv;  // (token, row) pairs
    const int rows = p.E + 1;
    const int t = unit / rows, row = unit - t * rows;
    if (t >= p.T) return;
    if (row < p.E) {
      const size_t esz = p.router_dtype == 1 ? 2 : 4;
      const void *wrow = static_cast<const uint8_t *>(p.router) + (size_t)row * p.H * esz;
      const float d = row_dot<XS>(wrow, p.router_dtype, p.H, p.x, xl, t);
      if (lane_id() == 0) p.logits[(size_t)t * p.E + row] = d;
    } else {
      const float d = row_dot<XS>(p.gvec, p.gate_dtype, p.H, p.x, xl, t);
      if (lane_id() == 0) p.sigma[t] = 1.0f / (1.0f + expf(-d));
    }
    return;
  }
  if constexpr (BITS_S != 0) {
    const int sw = (blk - p.n_router_blocks) * (kBlock / 64) + wv;
    if (sw >= p.n_shared_waves) return;
    gateup_wave<BITS_S, NCH_S, NPASS_S, XS>(p.shared_rec, p.soff, p.H, p.I,
                                            sw * p.shared_rows_per_wave, true, p.x, xl,
                                            p.h_shared);
  }
}

// ---------------------------------------------------------------------------
// stand-alone top-K (one wave per token)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_topk(TopkParams p) {
  const int t = blockIdx.x;
  const TopK r = wave_topk(p.logits + (size_t)t * p.E, p.E, p.K, p.renorm);
  write_topk(r, p.K, p.idx + (size_t)t * p.K, p.w + (size_t)t * p.K);
}

// ---------------------------------------------------------------------------
// K2: gate/up for a list of experts
// ---------------------------------------------------------------------------
template <int BITS, int NCH, int NPASS, int XS>
__global__ __launch_bounds__(kBlock) void k_gateup(GateUpParams p) {
  const int wave = wave_uniform(blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6));
  const int slot = wave / p.waves_per_expert;
  if (slot >= p.n) return;
  const int wie = wave - slot * p.waves_per_expert;
  int id;
  if (p.ids) {
    id = wave_uniform(p.ids[slot]);
  } else {
    const TopK t = wave_topk(p.logits, p.E, p.K, p.renorm);
    id = wave_uniform(pick_idx(t, slot));
    if (wave == 0) write_topk(t, p.K, p.idx_out, p.w_out);
  }
  const bool shared = id == kSharedId;
  const bool valid = shared ? (p.shared_ok != 0) : (id >= 0 && id < p.E);
  const uint8_t *rec = shared ? p.shared_rec : p.experts + (size_t)(valid ? id : 0) * p.stride;
  gateup_wave<BITS, NCH, NPASS, XS>(rec, shared ? p.soff : p.off, p.H, p.I,
                                    wie * p.rows_per_wave, valid, p.x, nullptr,
                                    p.h_out + (size_t)slot * p.I);
}

// ---------------------------------------------------------------------------
// K3: down projection
// ---------------------------------------------------------------------------
// one expert, rows [row0, row0 + NPASS*rpp): issue the loads
template <int BITS, int NCH, int NPASS>
__device__ __forceinline__ void down_load(const uint8_t *rec, const RecOffsets &off, int H,
                                          const RowMap &m, int row0, bool valid,
                                          uint4 (&q)[NPASS][NCH], uint32_t (&sb)[NPASS][NCH]) {
  const uint32_t *dc = reinterpret_cast<const uint32_t *>(rec + off.down_codes);
  const uint32_t *ds = reinterpret_cast<const uint32_t *>(rec + off.down_sb);
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int r = row0 + p * m.rpp + m.rip;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = m.li + (j << m.lg);
      if (valid && r < H && c < m.cpr) {
        q[p][j] = *reinterpret_cast<const uint4 *>(dc + (size_t)r * m.wpr + (size_t)c * 4);
        sb[p][j] = ds[(size_t)r * m.gpr + chunk_group<BITS>(c)];
      } else {
        q[p][j] = make_uint4(0, 0, 0, 0);
        sb[p][j] = 0;
      }
    }
  }
}

// weighted partial sums of one expert into acc[p]
template <int BITS, int NCH, int NPASS>
__device__ __forceinline__ void down_accumulate(const float *hin, const RowMap &m, bool valid,
                                                float wgt, const uint4 (&q)[NPASS][NCH],
                                                const uint32_t (&sb)[NPASS][NCH],
                                                float (&acc)[NPASS]) {
  XStage<BITS, true> xs[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = m.li + (j << m.lg);
    if (c < m.cpr) {
      float v[ChunkGeom<BITS>::kCols];
      load_x_chunk<BITS, XS_F32>(hin, nullptr, c * ChunkGeom<BITS>::kCols, v);
      stage_chunk<BITS>(v, xs[j]);
    }
  }
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = m.li + (j << m.lg);
      if (c < m.cpr) {
        const float d = chunk_dot<BITS>(q[p][j], xs[j]);
        part = fmaf(bf_lo(sb[p][j]), d, fmaf(bf_hi(sb[p][j]), xs[j].xs, part));
      }
    }
    acc[p] = valid ? fmaf(wgt, part, acc[p]) : __builtin_nanf("");
  }
}

// COMBINE: out = h_res + sum_k w_k y_k + sigma * y_shared for rows of a wave
// ([openclawradar] "Metal compute shaders": MoE combine + residual + sigmoid
// gate fused in one pass).  The weights are applied before the row reduction
// (the reduction is linear).  SHARED_IN: the shared expert has the routed
// width and is computed here; otherwise p.h_shared is null and p.y (if set)
// holds its precomputed down output.
template <int BITS, int NCH, int NPASS, int MAXK, bool SHARED_IN>
__global__ __launch_bounds__(kBlock) void k_down_combine(DownParams p) {
  const int wave = wave_uniform(blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6));
  const RowMap m = row_map<BITS>(p.I);
  const int row0 = wave * p.rows_per_wave;
  if (row0 >= p.H) return;

  int ids[MAXK];
  float wk[MAXK];
#pragma unroll
  for (int k = 0; k < MAXK; ++k) {
    ids[k] = k < p.K ? wave_uniform(p.idx[k]) : -2;
    wk[k] = k < p.K ? p.w[k] : 0.f;
  }
  uint4 q[MAXK][NPASS][NCH];
  uint32_t sb[MAXK][NPASS][NCH];
#pragma unroll
  for (int k = 0; k < MAXK; ++k) {
    const bool v = k < p.K && ids[k] >= 0 && ids[k] < p.E;
    down_load<BITS, NCH, NPASS>(p.experts + (size_t)(v ? ids[k] : 0) * p.stride, p.off, p.H, m,
                                row0, v, q[k], sb[k]);
  }
  uint4 qs[NPASS][NCH];
  uint32_t sbs[NPASS][NCH];
  if constexpr (SHARED_IN) down_load<BITS, NCH, NPASS>(p.shared_rec, p.soff, p.H, m, row0, true, qs, sbs);

  float acc[NPASS];
#pragma unroll
  for (int i = 0; i < NPASS; ++i) acc[i] = 0.f;
#pragma unroll
  for (int k = 0; k < MAXK; ++k) {
    if (k < p.K) {
      const bool v = ids[k] >= 0 && ids[k] < p.E;
      down_accumulate<BITS, NCH, NPASS>(p.h_routed + (size_t)k * p.I, m, v, wk[k], q[k], sb[k], acc);
    }
  }
  const float sig = p.sigma[0];
  if constexpr (SHARED_IN) down_accumulate<BITS, NCH, NPASS>(p.h_shared, m, true, sig, qs, sbs, acc);
#pragma unroll
  for (int i = 0; i < NPASS; ++i) {
    const float s = seg_sum(acc[i], m.lg);
    const int r = row0 + i * m.rpp + m.rip;
    if (m.li == 0 && r < p.H) {
      float o = p.h_res[r] + s;
      if constexpr (!SHARED_IN) {
        if (p.y) o = fmaf(sig, p.y[r], o);
      }
      p.out[r] = o;
    }
  }
}

// Y: y[slot][o] = W_down(ids[slot]) h[slot] for one expert per wave
template <int BITS, int NCH, int NPASS>
__global__ __launch_bounds__(kBlock) void k_down_y(DownParams p) {
  const int wave = wave_uniform(blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6));
  const int slot = wave / p.waves_per_expert;
  if (slot >= p.n) return;
  const int wie = wave - slot * p.waves_per_expert;
  const RowMap m = row_map<BITS>(p.I);
  const int row0 = wie * p.rows_per_wave;
  // a null id list selects the shared expert for every slot
  const int id = p.ids ? wave_uniform(p.ids[slot]) : kSharedId;
  const bool shared = id == kSharedId;
  const bool valid = shared ? (p.shared_ok != 0) : (id >= 0 && id < p.E);
  const uint8_t *rec = shared ? p.shared_rec : p.experts + (size_t)(valid ? id : 0) * p.stride;
  uint4 q[NPASS][NCH];
  uint32_t sb[NPASS][NCH];
  down_load<BITS, NCH, NPASS>(rec, shared ? p.soff : p.off, p.H, m, row0, valid, q, sb);
  float acc[NPASS];
#pragma unroll
  for (int i = 0; i < NPASS; ++i) acc[i] = 0.f;
  down_accumulate<BITS, NCH, NPASS>(p.h + (size_t)slot * p.I, m, valid, 1.0f, q, sb, acc);
#pragma unroll
  for (int i = 0; i < NPASS; ++i) {
    const float s = seg_sum(acc[i], m.lg);
    const int r = row0 + i * m.rpp + m.rip;
    if (m.li == 0 && r < p.H) p.y[(size_t)slot * p.H + r] = s;
  }
}

// ---------------------------------------------------------------------------
// elementwise combine (stand-alone entry point)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_combine(CombineParams p) {
  const int o = blockIdx.x * kBlock + threadIdx.x;
  if (o >= p.H) return;
  float acc = p.h_res[o];
  for (int k = 0; k < p.K; ++k) acc = fmaf(p.w[k], p.y[(size_t)k * p.H + o], acc);
  acc = fmaf(p.sigma[0], p.y_shared[o], acc);
  p.out[o] = acc;
}

// ---------------------------------------------------------------------------
// synthetic weights: SplitMix64 used counter-style (Steele, Lea and Flood,
// OOPSLA 2014), see moe_fill_experts in include/moe.h
// ---------------------------------------------------------------------------
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kRoot = 0x6D6F652D67656E31ull;

__device__ __forceinline__ uint64_t sm_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
__device__ __forceinline__ uint64_t sm_out(uint64_t key, uint64_t i) {
  return sm_mix(key + (i + 1) * kGamma);
}

// fp64 -> bf16 bits, round to nearest even from the full significand
__device__ __forceinline__ uint32_t f64_to_bf16(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t sign = (uint32_t)(b >> 63);
  if ((b << 1) == 0) return sign << 15;
  const int e = (int)((b >> 52) & 0x7FF);
  const uint64_t m = (b & ((1ull << 52) - 1)) | (1ull << 52);
  uint64_t keep = m >> 45;
  const uint64_t rem = m & ((1ull << 45) - 1);
  const uint64_t half = 1ull << 44;
  if (rem > half || (rem == half && (keep & 1))) ++keep;
  int exp = e - 1023 + 127;
  if (keep == 256) {
    keep = 128;
    ++exp;
  }
  return (sign << 15) | ((uint32_t)exp << 7) | (uint32_t)(keep & 0x7F);
}

__device__ __forceinline__ uint32_t uniform_bf16(uint32_t u24, double lo, double hi) {
  const double t = ((double)u24 + 0.5) * (1.0 / 16777216.0);
  const double d = __dsub_rn(hi, lo);
  const double v = __dadd_rn(lo, __dmul_rn(d, t));
  return f64_to_bf16(v);
}

__global__ __launch_bounds__(kBlock) void k_fill(FillParams p) {
  const int j = blockIdx.y;
  uint8_t *rec = p.dst + (size_t)j * p.stride;
  const uint64_t ng = (uint64_t)p.I * p.H * p.bits / 32;  // words of gate (= up)
  const uint64_t nd = ng;                                  // words of down
  const uint64_t gg = (uint64_t)p.I * (p.H / 64);          // sb words of gate (= up)
  const uint64_t gd = (uint64_t)p.H * (p.I / 64);          // sb words of down
  const uint64_t n_units[6] = {ng / 2, ng / 2, nd / 2, gg, gg, gd};
  const size_t offs[6] = {p.off.gate_codes, p.off.up_codes, p.off.down_codes,
                          p.off.gate_sb, p.off.up_sb, p.off.down_sb};
  uint64_t base = sm_out(sm_out(sm_out(kRoot, p.seed), (uint64_t)p.layer),
                         (uint64_t)(p.first_expert + j));
  uint64_t total = 0;
  for (int s = 0; s < 6; ++s) total += n_units[s];
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t u = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += stride) {
    int s = 0;
    uint64_t i = u;
    while (i >= n_units[s]) {
      i -= n_units[s];
      ++s;
    }
    const uint64_t key = sm_out(base, (uint64_t)s);
    const uint64_t r = sm_out(key, i);
    if (s < 3) {
      uint2 *dst = reinterpret_cast<uint2 *>(rec + offs[s]) + i;
      *dst = make_uint2((uint32_t)r, (uint32_t)(r >> 32));
    } else {
      const uint32_t us = (uint32_t)(r >> 40);
      const uint32_t ub = (uint32_t)((r >> 16) & 0xFFFFFFu);
      const uint32_t sbits = uniform_bf16(us, p.scale_lo, p.scale_hi);
      const uint32_t bbits = uniform_bf16(ub, p.bias_lo, p.bias_hi);
      reinterpret_cast<uint32_t *>(rec + offs[s])[i] = sbits | (bbits << 16);
    }
  }
}

__global__ __launch_bounds__(kBlock) void k_zero(uint8_t *ptr, size_t bytes) {
  const size_t n16 = bytes / 16;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    reinterpret_cast<uint4 *>(ptr)[i] = make_uint4(0, 0, 0, 0);
  const size_t tail = bytes - n16 * 16;
  if (blockIdx.x == 0 && threadIdx.x < tail) ptr[n16 * 16 + threadIdx.x] = 0;
}

__global__ __launch_bounds__(kBlock) void k_copy_f32(float *dst, const float *src, int n) {
  const int i = blockIdx.x * kBlock + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static int nch_for(int cols, int bits) {
  const int cpr = cols * bits / 128;
  const int lpr = cpr >= 64 ? 64 : (1 << ceil_log2(cpr));
  const int nch = (cpr + lpr - 1) / lpr;
  return nch <= 1 ? 1 : (nch <= 2 ? 2 : 4);
}
static int rpp_for(int cols, int bits) {
  const int cpr = cols * bits / 128;
  int lg = ceil_log2(cpr);
  if (lg > 6) lg = 6;
  return 64 >> lg;
}

#define MOE_DISPATCH_NCH(nch, ...) \
  switch (nch) {                   \
    case 1: { constexpr int NCH_ = 1; __VA_ARGS__; } break; \
    case 2: { constexpr int NCH_ = 2; __VA_ARGS__; } break; \
    default: { constexpr int NCH_ = 4; __VA_ARGS__; } break; \
  }

// rows of the shared expert per wave in K1
constexpr int kHeadSharedPass = 2;

hipError_t launch_head(const HeadParams &p0, hipStream_t s) {
  HeadParams p = p0;
  if (p.n_shared_waves > 0) {  // size the shared-expert part of the grid
    p.shared_rows_per_wave = kHeadSharedPass * rpp_for(p.H, p.bits_shared);
    p.n_shared_waves = (p.I + p.shared_rows_per_wave - 1) / p.shared_rows_per_wave;
  }
  const int rows = p.E + 1;
  p.n_router_blocks = (p.T * rows + 3) / 4;
  const int nsb = p.n_shared_waves > 0 ? (p.n_shared_waves + 3) / 4 : 0;
  const dim3 grid(p.n_router_blocks + nsb);
  const size_t lds = p.xsrc == XS_NORM ? (size_t)p.H * sizeof(float) : 0;
  const int bs = p.n_shared_waves > 0 ? p.bits_shared : 0;
  const int nch = bs ? nch_for(p.H, bs) : 1;
#define MOE_HEAD(XS)                                                                         \
  if (bs == 4) {                                                                             \
    MOE_DISPATCH_NCH(nch, hipLaunchKernelGGL((k_head<XS, 4, NCH_, kHeadSharedPass>), grid,   \
                                             dim3(kBlock), lds, s, p));                      \
  } else if (bs == 2) {                                                                      \
    MOE_DISPATCH_NCH(nch, hipLaunchKernelGGL((k_head<XS, 2, NCH_, kHeadSharedPass>), grid,   \
                                             dim3(kBlock), lds, s, p));                      \
  } else {                                                                                   \
    hipLaunchKernelGGL((k_head<XS, 0, 1, 1>), grid, dim3(kBlock), lds, s, p);                \
  }
  if (p.xsrc == XS_BF16) {
    MOE_HEAD(XS_BF16)
  } else if (p.xsrc == XS_F32) {
    MOE_HEAD(XS_F32)
  } else {
    MOE_HEAD(XS_NORM)
  }
#undef MOE_HEAD
  return hipGetLastError();
}

hipError_t launch_topk(const TopkParams &p, hipStream_t s) {
  hipLaunchKernelGGL(k_topk, dim3(p.T), dim3(64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gateup(const GateUpParams &p0, hipStream_t s) {
  GateUpParams p = p0;
  const int nch = nch_for(p.H, p.bits);
  const int rpp = rpp_for(p.H, p.bits);
  // about four rows per wave on wide rows, one pass on packed short rows
  const int npass = rpp >= 4 ? 1 : (p.I >= 4 * 64 ? 4 : 2);
  p.rows_per_wave = npass * rpp;
  p.waves_per_expert = (p.I + p.rows_per_wave - 1) / p.rows_per_wave;
  const int waves = p.waves_per_expert * p.n;
  const dim3 grid((waves + 3) / 4);
#define MOE_GU(BITS, XS)                                                                        \
  MOE_DISPATCH_NCH(nch, if (npass == 1) {                                                      \
    hipLaunchKernelGGL((k_gateup<BITS, NCH_, 1, XS>), grid, dim3(kBlock), 0, s, p);            \
  } else if (npass == 2) {                                                                     \
    hipLaunchKernelGGL((k_gateup<BITS, NCH_, 2, XS>), grid, dim3(kBlock), 0, s, p);            \
  } else {                                                                                     \
    hipLaunchKernelGGL((k_gateup<BITS, NCH_, 4, XS>), grid, dim3(kBlock), 0, s, p);            \
  })
  if (p.bits == 4) {
    if (p.xsrc == XS_BF16) { MOE_GU(4, XS_BF16) } else { MOE_GU(4, XS_F32) }
  } else {
    if (p.xsrc == XS_BF16) { MOE_GU(2, XS_BF16) } else { MOE_GU(2, XS_F32) }
  }
#undef MOE_GU
  return hipGetLastError();
}

hipError_t launch_down(const DownParams &p0, hipStream_t s) {
  DownParams p = p0;
  const int bits = p.bits_r;
  const int nch = nch_for(p.I, bits);
  const int rpp = rpp_for(p.I, bits);
  const int npass = rpp >= 8 ? 1 : 2;
  p.rows_per_wave = npass * rpp;
  if (p.combine) {
    const bool shared_in = p.h_shared != nullptr;
    const int waves = (p.H + p.rows_per_wave - 1) / p.rows_per_wave;
    const dim3 grid((waves + 3) / 4);
    const int maxk = p.K <= 2 ? 2 : (p.K <= 4 ? 4 : 8);
#define MOE_DC(BITS, MAXK, SIN)                                                                  \
  MOE_DISPATCH_NCH(nch, if (npass == 1) {                                                       \
    hipLaunchKernelGGL((k_down_combine<BITS, NCH_, 1, MAXK, SIN>), grid, dim3(kBlock), 0, s, p); \
  } else {                                                                                      \
    hipLaunchKernelGGL((k_down_combine<BITS, NCH_, 2, MAXK, SIN>), grid, dim3(kBlock), 0, s, p); \
  })
#define MOE_DC_K(BITS, SIN)        \
  if (maxk == 2) {                 \
    MOE_DC(BITS, 2, SIN)           \
  } else if (maxk == 4) {          \
    MOE_DC(BITS, 4, SIN)           \
  } else {                         \
    MOE_DC(BITS, 8, SIN)           \
  }
    if (bits == 4) {
      if (shared_in) { MOE_DC_K(4, true) } else { MOE_DC_K(4, false) }
    } else {
      if (shared_in) { MOE_DC_K(2, true) } else { MOE_DC_K(2, false) }
    }
#undef MOE_DC_K
#undef MOE_DC
  } else {
    p.waves_per_expert = (p.H + p.rows_per_wave - 1) / p.rows_per_wave;
    const int waves = p.waves_per_expert * p.n;
    const dim3 grid((waves + 3) / 4);
#define MOE_DY(BITS)                                                                  \
  MOE_DISPATCH_NCH(nch, if (npass == 1) {                                            \
    hipLaunchKernelGGL((k_down_y<BITS, NCH_, 1>), grid, dim3(kBlock), 0, s, p);      \
  } else {                                                                           \
    hipLaunchKernelGGL((k_down_y<BITS, NCH_, 2>), grid, dim3(kBlock), 0, s, p);      \
  })
    if (bits == 4) { MOE_DY(4) } else { MOE_DY(2) }
#undef MOE_DY
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams &p, hipStream_t s) {
  hipLaunchKernelGGL(k_combine, dim3((p.H + kBlock - 1) / kBlock), dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_fill(const FillParams &p, hipStream_t s) {
  const dim3 grid(1024, p.n);
  hipLaunchKernelGGL(k_fill, grid, dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_zero(void *ptr, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  size_t blocks = (bytes / 16 + kBlock - 1) / kBlock;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_zero, dim3((unsigned)blocks), dim3(kBlock), 0, s,
                     static_cast<uint8_t *>(ptr), bytes);
  return hipGetLastError();
}

hipError_t launch_copy_f32(float *dst, const float *src, int n, hipStream_t s) {
  hipLaunchKernelGGL(k_copy_f32, dim3((n + kBlock - 1) / kBlock), dim3(kBlock), 0, s, dst, src, n);
  return hipGetLastError();
}

}  // namespace moe_impl
