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
  const float4 k4 = reinterpret_cast<const float4 *>(p.k + (size_t)sh * p.d_k)[li];
  const float4 q4 = reinterpret_cast<const float4 *>(p.q + (size_t)sh * p.d_k)[li];
  const float a = p.alpha[sh], b = p.beta[sh];
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
