// moe_gdn.hip -- gfx950 kernel of the linear-attention decode step: the
// gated delta rule on a per-head state matrix ([openclawradar] "Accelerate
// BLAS for linear attention"; [a2a-fr] "Technical deep dive / 4": 64 heads,
// 128x128 state, updated by a scale, a matrix-vector product and a rank-1
// update).  Per sequence and head, with S stored as d_v rows of d_k columns:
//     S <- alpha S;  u = S k;  S <- S + beta (v - u) k^T;  o = S q.
// Row i of the result depends on row i of S only, so one pass reads and
// writes each row once: the step is bound by the state's HBM traffic.
#include "moe_device.h"

#include <stdint.h>

namespace moe_impl {

namespace {

__device__ __forceinline__ float dot4(const float4 &a, const float4 &b) {
  return fmaf(a.w, b.w, fmaf(a.z, b.z, fmaf(a.y, b.y, a.x * b.x)));
}

}  // namespace

// A row of d_k values is held by d_k / 4 lanes (16 bytes each); a wave takes
// 64 / (d_k / 4) rows per pass and kGdnPasses passes (loads of all passes
// before the arithmetic).  One pass, the most waves, measured fastest for
// 64 heads of 128 x 128 (3.6 us per step against 4.0 for two passes and 4.3
// for four).
constexpr int kGdnPasses = 1;

__global__ __launch_bounds__(kBlock) void k_gdn_step(GdnParams p) {
  const int wave = blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6);
  const int lane = lane_id();
  const int lpr = p.d_k >> 2;              // lanes per row (power of two, <= 64)
  const int lg = 31 - __clz(lpr);
  const int li = lane & (lpr - 1), rip = lane >> lg;
  const int rpp = 64 >> lg;                // rows per pass
  const int rpw = rpp * kGdnPasses;        // rows per wave
  const int wph = (p.d_v + rpw - 1) / rpw;  // waves per head
  const int sh = wave / wph;               // sequence * n_heads + head
  if (sh >= p.n_sh) return;                // wave-uniform
  const int row0 = (wave - sh * wph) * rpw;
  float4 k4 = reinterpret_cast<const float4 *>(p.k + (size_t)sh * p.d_k)[li];
  float4 q4 = reinterpret_cast<const float4 *>(p.q + (size_t)sh * p.d_k)[li];
  float a = p.alpha[sh], b = p.beta[sh];
  if (p.prep) {  // uniform: raw projections and gate logits of the block
    const float rq = 1.0f / sqrtf(seg_sum(dot4(q4, q4), lg) + 1e-6f);
    const float rk = 1.0f / sqrtf(seg_sum(dot4(k4, k4), lg) + 1e-6f);
    q4 = make_float4(q4.x * rq, q4.y * rq, q4.z * rq, q4.w * rq);
    k4 = make_float4(k4.x * rk, k4.y * rk, k4.z * rk, k4.w * rk);
    a = 1.0f / (1.0f + expf(-a));
    b = 1.0f / (1.0f + expf(-b));
  }
  float *S = p.state + (size_t)sh * p.d_v * p.d_k;
  float4 s4[kGdnPasses];
  float vi[kGdnPasses];
#pragma unroll
  for (int ps = 0; ps < kGdnPasses; ++ps) {
    const int r = row0 + ps * rpp + rip;
    const int rr = r < p.d_v ? r : 0;      // rows past the end load row 0
    s4[ps] = reinterpret_cast<const float4 *>(S + (size_t)rr * p.d_k)[li];
    vi[ps] = p.v[(size_t)sh * p.d_v + rr];
  }
#pragma unroll
  for (int ps = 0; ps < kGdnPasses; ++ps) {
    const int r = row0 + ps * rpp + rip;
    float4 x = s4[ps];
    x.x *= a;  // scale
    x.y *= a;
    x.z *= a;
    x.w *= a;
    const float u = seg_sum(dot4(x, k4), lg);  // u_r = (alpha S k)_r
    const float c = b * (vi[ps] - u);
    x.x = fmaf(c, k4.x, x.x);                       // rank-1 delta update
    x.y = fmaf(c, k4.y, x.y);
    x.z = fmaf(c, k4.z, x.z);
    x.w = fmaf(c, k4.w, x.w);
    const float o = seg_sum(dot4(x, q4), lg);  // o_r = (S_new q)_r
    if (r < p.d_v) {
      reinterpret_cast<float4 *>(S + (size_t)r * p.d_k)[li] = x;
      if (li == 0) p.out[(size_t)sh * p.d_v + r] = o;
    }
  }
}

// ---------------------------------------------------------------------------
// the block's projections.  Every workgroup normalises h into LDS (two passes:
// the sum of squares, then the scaled values in the padded chunk layout of
// the fp32 dot path); each wave takes rows_per_wave rows of one projection
// matrix and requests them before the normalisation, so that their latency
// overlaps it.
// ---------------------------------------------------------------------------
template <int BITS, int WAVES>
__device__ __forceinline__ void norm_to_lds(const float *h, int H, float *xl) {
  constexpr int kThreads = 64 * WAVES;
  constexpr int kSteps = kMaxDim / (4 * kThreads);
  __shared__ float red[WAVES];
  float4 hv[kSteps];
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int c = (i * kThreads + (int)threadIdx.x) * 4;
    hv[i] = *reinterpret_cast<const float4 *>(h + (c < H ? c : 0));
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int c = (i * kThreads + (int)threadIdx.x) * 4;
    if (c < H) {
      ss = fmaf(hv[i].x, hv[i].x, ss);
      ss = fmaf(hv[i].y, hv[i].y, ss);
      ss = fmaf(hv[i].z, hv[i].z, ss);
      ss = fmaf(hv[i].w, hv[i].w, ss);
    }
  }
  ss = seg_sum(ss, 6);
  if (lane_id() == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < WAVES; ++i) tot += red[i];
  const float r = 1.0f / sqrtf(tot / (float)H + 1e-6f);
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int c = (i * kThreads + (int)threadIdx.x) * 4;
    // H is a multiple of 64, so a chunk's lanes agree on c < H
    if (c < H)
      lds_put_chunk4<BITS>(xl, c, make_float4(hv[i].x * r, hv[i].y * r, hv[i].z * r, hv[i].w * r));
  }
  __syncthreads();
}

constexpr int kGdnInWaves = 8;

// The grid holds as many workgroups as fit the CUs at once; each normalises
// h once and its waves loop over units (rows_per_wave rows of one matrix),
// unit u of a wave followed by u + (waves in the grid), each unit's rows
// requested before the previous unit is computed.  (One unit per wave took
// three rounds of workgroups at 4,096 rows per matrix, each round paying the
// normalisation again: 19.2 us per block.)
template <int BITS, int NCH, int NPASS>
__global__ __launch_bounds__(64 * kGdnInWaves) void k_gdn_in(GdnInParams p) {
  extern __shared__ float xl[];
  const int wave0 = wave_uniform(blockIdx.x * kGdnInWaves + (threadIdx.x >> 6));
  const int stride = (int)gridDim.x * kGdnInWaves;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    p.one_idx[0] = 0;
    p.one_w[0] = 1.0f;
    p.zero_sigma[0] = 0.0f;
  }
  // unit -> matrix (0 q, 1 k, 2 v, 3 the gate rows) and its first row
  const int rpw = p.rows_per_wave;
  const int wpm = (p.D + rpw - 1) / rpw;
  const int n_units = 3 * wpm + (2 * p.n_heads + rpw - 1) / rpw;
  const RowMap m = row_map<BITS>(p.H);
  struct Unit {
    int mat, row0, rows;
    const uint8_t *rec;
    RecOffsets off;
  };
  auto unit_of = [&](int u) {
    Unit r;
    r.mat = u / wpm < 3 ? u / wpm : 3;
    r.row0 = (u - r.mat * wpm) * rpw;
    r.rows = r.mat < 3 ? p.D : 2 * p.n_heads;
    r.off = p.off;
    r.off.down_codes = (r.mat & 1) ? p.off.up_codes : p.off.gate_codes;
    r.off.down_sb = (r.mat & 1) ? p.off.up_sb : p.off.gate_sb;
    r.rec = r.mat < 2 ? p.rec_qko : p.rec_vab;
    return r;
  };
  // two tiles in turn: unit u is computed while unit u + stride is on its
  // way.  The loop is unrolled by two so that a tile is refilled only after
  // its unit was computed: copying the prefetched tile into the current one
  // waited for its loads at the end of every unit (60-layer stack with the
  // block: 44.0 -> 43.3 us per layer, this kernel 17.0 -> 16.0 us).  Two
  // units ahead (three tiles) spills at two workgroups per CU, since each
  // lane keeps its x columns in registers: 26 us.
  DnTile<BITS, NCH, NPASS> ta, tb;
  auto fetch = [&](DnTile<BITS, NCH, NPASS> &t, int v) {
    if (v < n_units) {  // wave-uniform
      const Unit n = unit_of(v);
      const bool ok = n.row0 < n.rows;
      down_load(t, n.rec, n.off, ok ? n.rows : 1, m, ok ? n.row0 : 0);
    }
  };
  int u = wave0;
  fetch(ta, u);
  norm_to_lds<BITS, kGdnInWaves>(p.h, p.H, xl);
  XStage<BITS, true> xs[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = m.li + (j << m.lg);
    xs[j] = make_stage<BITS, XS_LDSPAD>(nullptr, xl, c < m.cpr ? c : 0);
  }
  // fill `next` with unit u + stride, then compute unit u from `cur`
  auto step = [&](DnTile<BITS, NCH, NPASS> &cur, DnTile<BITS, NCH, NPASS> &next) {
    fetch(next, u + stride);
    const Unit cu = unit_of(u);
    if (cu.row0 < cu.rows) {
      float acc[NPASS];
#pragma unroll
      for (int i = 0; i < NPASS; ++i) acc[i] = 0.f;
      down_accumulate_staged<BITS, NCH, NPASS>(xs, m, cu.rows, cu.row0, true, 1.0f, cur, acc);
      float *out = p.proj + (size_t)cu.mat * p.D;
#pragma unroll
      for (int i = 0; i < NPASS; ++i) {
        const float sum = seg_sum(acc[i], m.lg);
        const int r = cu.row0 + i * m.rpp + m.rip;
        if (m.li == 0 && r < cu.rows) out[r] = sum;
      }
    }
    u += stride;
  };
  while (u < n_units) {  // wave-uniform
    step(ta, tb);
    if (u >= n_units) break;
    step(tb, ta);
  }
}

hipError_t launch_gdn_in(const GdnInParams &p0, hipStream_t s) {
  GdnInParams p = p0;
  const int nch = nch_for(p.H, p.bits);
  const int rpp = rpp_for(p.H, p.bits);
  // one pass of rows per unit: the waves loop over units, and the lighter
  // tile lets two workgroups share a CU
  const int npass = 1;
  p.rows_per_wave = npass * rpp;
  const int wpm = (p.D + p.rows_per_wave - 1) / p.rows_per_wave;
  const int waves = 3 * wpm + (2 * p.n_heads + p.rows_per_wave - 1) / p.rows_per_wave;
  // at most the workgroups that fit the CUs at once: two per CU, one for the
  // variants with more than 128 VGPRs (four 4-bit or two 2-bit chunks per lane)
  const int per_cu = (nch >= 4 || (p.bits == 2 && nch >= 2)) ? 1 : 2;
  int blocks = (waves + kGdnInWaves - 1) / kGdnInWaves;
  if (blocks > kCUs * per_cu) blocks = kCUs * per_cu;
  const dim3 grid(blocks);
  const int nc = 128 / p.bits;
  const size_t lds = (size_t)(p.H / nc) * (nc + kLdsPad) * sizeof(float);
#define MOE_GI(BITS)                                                                            \
  do {                                                                                          \
    if (nch == 1 && npass == 1) MOE_LAUNCH((k_gdn_in<BITS, 1, 1>), grid, dim3(64 * kGdnInWaves), lds, s, p); \
    else if (nch == 1) MOE_LAUNCH((k_gdn_in<BITS, 1, 2>), grid, dim3(64 * kGdnInWaves), lds, s, p);          \
    else if (nch == 2 && npass == 1) MOE_LAUNCH((k_gdn_in<BITS, 2, 1>), grid, dim3(64 * kGdnInWaves), lds, s, p); \
    else if (nch == 2) MOE_LAUNCH((k_gdn_in<BITS, 2, 2>), grid, dim3(64 * kGdnInWaves), lds, s, p);          \
    else MOE_LAUNCH((k_gdn_in<BITS, 4, 1>), grid, dim3(64 * kGdnInWaves), lds, s, p);                       \
  } while (0)
  if (p.bits == 4) MOE_GI(4);
  else MOE_GI(2);
#undef MOE_GI
  return hipGetLastError();
}

hipError_t launch_gdn_step(const GdnParams &p, hipStream_t s) {
  const int lpr = p.d_k / 4;
  int lg = 0;
  while ((1 << lg) < lpr) ++lg;
  const int rpw = (64 >> lg) * kGdnPasses;
  const long waves = (long)p.n_sh * ((p.d_v + rpw - 1) / rpw);
  const dim3 grid((unsigned)((waves + 3) / 4));
  MOE_LAUNCH(k_gdn_step, grid, dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe_impl
