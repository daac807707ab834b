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
// converts when x is fp32.  x is staged once (a lane always sees the same
// input columns) and the bias term needs only the chunk sums of x.
//
// Memory mapping: a wave reads whole quantised rows with 128-bit loads, lane l
// taking 16-byte chunks l, l+64, ... of a row (rows shorter than 64 chunks are
// packed several to a wave), so every load instruction covers one contiguous
// run of up to 1 KiB.  Each wave issues all of its weight loads before it
// computes.  Rows are reduced with DPP.
#include "moe_device.h"

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

namespace moe_impl {

template <int XS, int BITS_S, int NCH_S, int NPASS_S>
__global__ __launch_bounds__(kBlock) void k_head(HeadParams p) {
  extern __shared__ float xl[];
  const int wv = wave_uniform(threadIdx.x >> 6);
  const int blk = wave_uniform(blockIdx.x);
  // waves per workgroup: two where every wave only reads its row (the 513
  // rows of a token then reach all 256 CUs), four with the norm prologue or
  // the shared expert's rows
  const int wpb = (int)(blockDim.x / 64);
  // the stack path normalises x in every workgroup: the router row is
  // requested first so that its latency overlaps the normalisation
  RowPre pre{};
  bool have_pre = false;
  // the dots of the rows are taken with h + u and scaled by the norm's
  // reciprocal when only dots read x here (no shared expert's rows)
  float rscale = 1.0f;
  if constexpr (XS == XS_NORM) {
    const int unit = blk * wpb + wv;
    const int row = unit - (unit / (p.E + 1)) * (p.E + 1);
    if (blk < p.n_router_blocks && unit < p.T * (p.E + 1) && row < p.E) {
      const size_t esz = p.router_dtype == 1 ? 2 : 4;
      pre = row_prefetch(static_cast<const uint8_t *>(p.router) + (size_t)row * p.H * esz,
                         p.router_dtype, p.H);
      have_pre = true;
    }
    if constexpr (BITS_S == 0) rscale = norm_prologue_scaled(p, xl);
    else norm_prologue(p, xl);
  }
  if (blk < p.n_router_blocks) {
    const int unit = blk * wpb + wv;  // (token, row) pairs, then one x stager per token
    const int rows = p.E + 1;
    if (unit >= p.T * rows) {
      const int st = unit - p.T * rows;
      if constexpr (XS == XS_BF16) {
        if (p.xs_pairs && st < p.T) {
          const void *xt = static_cast<const uint16_t *>(p.x) + (size_t)st * p.H;
          uint32_t *pairs = p.xs_pairs + (size_t)st * p.xs_pair_stride;
          float *sums = p.xs_sums + (size_t)st * p.xs_sum_stride;
          if (p.bits_routed == 4) write_xstage<4>(xt, p.H, pairs, sums);
          else write_xstage<2>(xt, p.H, pairs, sums);
        }
      }
      return;
    }
    const int t = unit / rows, row = unit - t * rows;
    if (t >= p.T) return;
    if (row < p.E) {
      const size_t esz = p.router_dtype == 1 ? 2 : 4;
      const void *wrow = static_cast<const uint8_t *>(p.router) + (size_t)row * p.H * esz;
      const float d = row_dot<XS>(wrow, p.router_dtype, p.H, p.x, xl, t, pre, have_pre) * rscale;
      if (lane_id() == 0) p.logits[(size_t)t * p.E + row] = d;
    } else {
      const float d = row_dot<XS>(p.gvec, p.gate_dtype, p.H, p.x, xl, t) * rscale;
      if (lane_id() == 0) p.sigma[t] = 1.0f / (1.0f + expf(-d));
    }
    return;
  }
  if constexpr (BITS_S != 0) {
    const int sw = (blk - p.n_router_blocks) * wpb + wv;
    if (sw >= p.n_shared_waves) return;
    constexpr bool XF32 = XS != XS_BF16;
    const RowMap m = row_map<BITS_S>(p.H);
    const int row0 = sw * p.shared_rows_per_wave;
    XRaw<BITS_S, XS> xr[NCH_S];
#pragma unroll
    for (int j = 0; j < NCH_S; ++j) {
      const int c = m.li + (j << m.lg);
      xr[j] = load_raw<BITS_S, XS>(p.x, xl, c < m.cpr ? c : 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    GUTile<BITS_S, NCH_S, NPASS_S> tile;
    gu_load(tile, p.shared_rec, p.soff, m, p.I, row0);
    __builtin_amdgcn_sched_barrier(0);
    XStage<BITS_S, XF32> xs[NCH_S];
#pragma unroll
    for (int j = 0; j < NCH_S; ++j) xs[j] = stage_raw<BITS_S, XS>(xr[j]);
    gu_compute(tile, xs, m, p.I, row0, true, p.h_shared);
  }
}

// ---------------------------------------------------------------------------
// stand-alone top-K (one wave per token)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_topk(TopkParams p) {
  const int t = blockIdx.x;
  float v[kTopkNpl];
  topk_load(p.logits + (size_t)t * p.E, p.E, v);
  int e;
  float w;
  topk_select(v, p.E, p.K, p.renorm, e, w);
  topk_store(e, w, p.K, p.idx + (size_t)t * p.K, p.w + (size_t)t * p.K);
}

// ---------------------------------------------------------------------------
// K2: gate/up for a list of experts (explicit ids, or the top-K of the
// logits, computed by every workgroup)
// ---------------------------------------------------------------------------
// Expert tier: copy workgroup c moves its share of the down section (codes,
// then scale/bias words) of entry c / copy_blocks_per_entry from the record it
// is read from (host memory on a miss) into the entry's cache slot, so that
// the down kernel reads every record from device memory and the host link
// carries a missing record's down rows while its gate/up rows stream in.
constexpr int kCopyUnroll = 8;  // 16-byte words per thread in flight

__device__ __forceinline__ void copy_down_part(const GateUpParams &p, int c) {
  const int k = c / p.copy_blocks_per_entry;
  const int part = c - k * p.copy_blocks_per_entry;
  const uint64_t fill = wave_uniform_u64(p.rec_fill[k]);
  if (!fill) return;  // a hit: the slot already holds the record
  const uint8_t *src = reinterpret_cast<const uint8_t *>(wave_uniform_u64(p.rec_src[k]));
  uint8_t *dst = reinterpret_cast<uint8_t *>(fill);
  const size_t n_codes = (size_t)p.H * p.I * p.bits / 8 / 16;  // 16-byte words
  const size_t n_sb = (size_t)p.H * (p.I / kGroup) * 4 / 16;
  const size_t n = n_codes + n_sb;
  const size_t per = (n + p.copy_blocks_per_entry - 1) / p.copy_blocks_per_entry;
  const size_t w0 = (size_t)part * per, w1 = w0 + per < n ? w0 + per : n;
  for (size_t b = w0 + threadIdx.x; b < w1; b += (size_t)kBlock * kCopyUnroll) {
    uint4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const size_t i = b + (size_t)u * kBlock;
      const size_t off = i < n_codes ? p.off.down_codes + i * 16 : p.off.down_sb + (i - n_codes) * 16;
      if (i < w1) v[u] = *reinterpret_cast<const uint4 *>(src + off);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const size_t i = b + (size_t)u * kBlock;
      const size_t off = i < n_codes ? p.off.down_codes + i * 16 : p.off.down_sb + (i - n_codes) * 16;
      if (i < w1) *reinterpret_cast<uint4 *>(dst + off) = v[u];
    }
  }
}
template <int BITS, int NCH, int NPASS, int XS>
__global__ __launch_bounds__(kBlock) void k_gateup(GateUpParams p) {
  // each wave stages its own chunks of x (see gateup_x_in_lds)
  __shared__ TopkShare tsh;
  static_assert(kBlock / 64 == 4, "the selection is split over four waves");
  const int blk = wave_uniform(blockIdx.x);
  const int wv = wave_uniform(threadIdx.x >> 6);
  // The routed workgroups come first in the grid, so they are dispatched and
  // issue their logit loads ahead of the shared expert's: those need no
  // routing and stream the shared rows while the routed ones select experts
  // (q4 layer 20.36 -> 20.10 us per layer with this order)
  const int n_routed_blocks = (int)gridDim.x - p.n_shared_blocks - p.n_copy_blocks;
  if (blk >= n_routed_blocks + p.n_shared_blocks) {  // workgroup-uniform: a tier copy
    copy_down_part(p, blk - n_routed_blocks - p.n_shared_blocks);
    return;
  }
  const bool shared_blk = blk >= n_routed_blocks;
  const int wave = shared_blk ? (blk - n_routed_blocks) * (kBlock / 64) + wv
                              : blk * (kBlock / 64) + wv;
  const int slot = shared_blk ? 0 : wave / p.waves_per_expert;
  const int wie = shared_blk ? wave : wave - slot * p.waves_per_expert;
  const bool topk = !shared_blk && !p.ids;  // workgroup-uniform
  if (!topk && (shared_blk ? wie >= p.waves_per_expert : slot >= p.n)) return;

  // Routing: the four waves of the workgroup each take a quarter of the
  // logits, and after one barrier each merges the quarters' candidates.
  // Loads go out in the order they are needed (vmcnt counts in order):
  // logits, x, then the weights once the expert is known.
  float lv[4];
  const int npl = topk_npl(p.E);
  if (topk) {
    if (npl == 2) topk_part_load<2>(p.logits, p.E, wv, lv);
    else topk_part_load<4>(p.logits, p.E, wv, lv);
  }
  constexpr bool XF32 = XS != XS_BF16;
  const RowMap m = row_map<BITS>(p.H);
  const int row0 = wie * p.rows_per_wave;
  XStage<BITS, XF32> xs[NCH];
  XRaw<BITS, XS> xr[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = m.li + (j << m.lg);
    xr[j] = load_raw<BITS, XS>(p.x, nullptr, c < m.cpr ? c : 0);
  }
  __builtin_amdgcn_sched_barrier(0);

  int id;
  float *hout;
  int sel_e = -2;
  uint32_t sel_key = 0, top_key = 0;
  if (shared_blk) {
    id = kSharedId;
    hout = p.h_shared_out;
  } else {
    if (topk) {
      // the selection gates every routed load of the workgroup: issue it
      // ahead of the shared-expert waves computing on the same SIMD
      __builtin_amdgcn_s_setprio(3);
      if (npl == 2) topk_part_select<2>(lv, p.E, p.K, p.renorm, wv, tsh);
      else topk_part_select<4>(lv, p.E, p.K, p.renorm, wv, tsh);
      __syncthreads();
      if (slot >= p.n) return;
      topk_merge(tsh, p.E, p.K, sel_e, sel_key, top_key);
      __builtin_amdgcn_s_setprio(0);
      id = __builtin_amdgcn_readlane(sel_e, slot);
    } else {
      id = wave_uniform(p.ids[slot]);
    }
    hout = p.h_out + (size_t)slot * p.I;
  }
  // an entry whose record cannot be read at this width (an id out of range,
  // or the shared expert at another width) reads routed record 0 with the
  // routed geometry, so every load stays inside the records, and yields NaN
  const bool shared = id == kSharedId;
  const bool valid = shared ? (p.shared_ok != 0) : (id >= 0 && id < p.E);
  const bool from_shared = shared && valid;
  const uint8_t *rec = from_shared ? p.shared_rec : p.experts + (size_t)(valid && !shared ? id : 0) * p.stride;
  uint8_t *fill = nullptr;
  if (p.rec_src && !shared_blk && valid && !shared) {  // the tier's record of this entry
    rec = reinterpret_cast<const uint8_t *>(wave_uniform_u64(p.rec_src[slot]));
    fill = reinterpret_cast<uint8_t *>(wave_uniform_u64(p.rec_fill[slot]));
  }
  GUTile<BITS, NCH, NPASS> tile;
  gu_load(tile, rec, from_shared ? p.soff : p.off, m, p.I, row0);
  __builtin_amdgcn_sched_barrier(0);
  if (fill) gu_store(tile, fill, p.off, m, p.I, row0);
  // the first routed workgroup also reports the selection and its weights
  if (topk && blk == 0 && wv == 0)
    topk_store(sel_e, topk_merge_weight(tsh, p.K, p.renorm, sel_e, sel_key, top_key), p.K,
               p.idx_out, p.w_out);
#pragma unroll
  for (int j = 0; j < NCH; ++j) xs[j] = stage_raw<BITS, XS>(xr[j]);
  gu_compute(tile, xs, m, p.I, row0, valid, hout);
}

// K2 with x staged once per workgroup in LDS (XLds): the same work, for
// shapes where a wave's own chunks of x would outweigh its weight rows
template <int BITS, int NCH, int NPASS, int XS>
__global__ __launch_bounds__(kBlock) void k_gateup_xl(GateUpParams p) {
  // x of the workgroup (XLds layout), staged before the one barrier (every
  // workgroup has it: the x of a wave comes from the others' parts)
  extern __shared__ uint32_t xw[];
  __shared__ TopkShare tsh;
  constexpr bool XF32 = XS != XS_BF16;
  const int blk = wave_uniform(blockIdx.x);
  const int wv = wave_uniform(threadIdx.x >> 6);
  // The routed workgroups come first in the grid, so they are dispatched and
  // issue their logit loads ahead of the shared expert's: those need no
  // routing and stream the shared rows while the routed ones select experts
  // (q4 layer 20.36 -> 20.10 us per layer with this order)
  const int n_routed_blocks = (int)gridDim.x - p.n_shared_blocks - p.n_copy_blocks;
  if (blk >= n_routed_blocks + p.n_shared_blocks) {  // workgroup-uniform: a tier copy
    copy_down_part(p, blk - n_routed_blocks - p.n_shared_blocks);
    return;
  }
  const bool shared_blk = blk >= n_routed_blocks;
  const int wave = shared_blk ? (blk - n_routed_blocks) * (kBlock / 64) + wv
                              : blk * (kBlock / 64) + wv;
  const int slot = shared_blk ? 0 : wave / p.waves_per_expert;
  const int wie = shared_blk ? wave : wave - slot * p.waves_per_expert;
  const bool topk = !shared_blk && !p.ids;  // workgroup-uniform
  // a wave without rows still stages its part of x
  const bool active = shared_blk ? wie < p.waves_per_expert : slot < p.n;

  // Loads go out in the order they are needed (vmcnt counts in order): the
  // wave's quarter of the logits (routing workgroups), this thread's part of
  // x, then the weights as soon as the expert is known.
  float lv[4];
  const int npl = topk_npl(p.E);
  if (topk) {
    if (npl == 2) topk_part_load<2>(p.logits, p.E, wv, lv);
    else topk_part_load<4>(p.logits, p.E, wv, lv);
  }
  const RowMap m = row_map<BITS>(p.H);
  XPart<BITS, XS> xp;
  xpart_load(xp, p.x, p.H);
  const int row0 = wie * p.rows_per_wave;
  GUTile<BITS, NCH, NPASS> tile;
  bool valid = false;
  // a list entry may name the shared expert: it still writes its own slot
  float *const hout = shared_blk ? p.h_shared_out : p.h_out + (size_t)slot * p.I;
  uint8_t *fill = nullptr;
  auto issue = [&](int id) {
    // unreadable entries (see k_gateup) read routed record 0 and yield NaN
    const bool shared = id == kSharedId;
    valid = shared ? (p.shared_ok != 0) : (id >= 0 && id < p.E);
    const bool from_shared = shared && valid;
    const uint8_t *rec = from_shared ? p.shared_rec : p.experts + (size_t)(valid && !shared ? id : 0) * p.stride;
    if (p.rec_src && !shared_blk && valid && !shared) {  // the tier's record of this entry
      rec = reinterpret_cast<const uint8_t *>(wave_uniform_u64(p.rec_src[slot]));
      fill = reinterpret_cast<uint8_t *>(wave_uniform_u64(p.rec_fill[slot]));
    }
    gu_load(tile, rec, from_shared ? p.soff : p.off, m, p.I, row0);
  };
  if (!topk && active) issue(shared_blk ? kSharedId : wave_uniform(p.ids[slot]));
  __builtin_amdgcn_sched_barrier(0);
  // the selection gates every routed load of the workgroup: issue it ahead
  // of the shared-expert waves computing on the same SIMD
  if (topk) {
    __builtin_amdgcn_s_setprio(3);
    if (npl == 2) topk_part_select<2>(lv, p.E, p.K, p.renorm, wv, tsh);
    else topk_part_select<4>(lv, p.E, p.K, p.renorm, wv, tsh);
  }
  xpart_store(xp, xw, p.H);
  __syncthreads();
  if (!active) return;
  int sel_e = -2;
  uint32_t sel_key = 0, top_key = 0;
  if (topk) {
    topk_merge(tsh, p.E, p.K, sel_e, sel_key, top_key);
    __builtin_amdgcn_s_setprio(0);
    issue(__builtin_amdgcn_readlane(sel_e, slot));
  }
  __builtin_amdgcn_sched_barrier(0);
  // the first routed workgroup also reports the selection and its weights
  if (topk && blk == 0 && wv == 0)
    topk_store(sel_e, topk_merge_weight(tsh, p.K, p.renorm, sel_e, sel_key, top_key), p.K,
               p.idx_out, p.w_out);
  if (fill) gu_store(tile, fill, p.off, m, p.I, row0);
  XStage<BITS, XF32> xs[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = m.li + (j << m.lg);
    xs[j] = xlds_read<BITS, XF32>(xw, c < m.cpr ? c : 0);
  }
  gu_compute(tile, xs, m, p.I, row0, valid, hout);
}

// COMBINE: out = h_res + sum_k w_k y_k + sigma * y_shared for rows of a wave
// ([openclawradar] "Metal compute shaders": MoE combine + residual + sigmoid
// gate fused in one pass).  The weights are applied before the row reduction
// (the reduction is linear).  SHARED_IN: the shared expert has the routed
// width and is computed here; otherwise p.h_shared is null and p.y (if set)
// holds its precomputed down output.  WAVES: waves per workgroup; each
// workgroup stages all K + 1 SwiGLU vectors, so eight waves halve those L2
// reads per weight byte where the grid still gives every CU a workgroup.
// SPLIT: where the rows give fewer waves than that, two waves share each set
// of rows, one taking the first half of the experts (the shared one first)
// and the other the rest; their partial sums meet in LDS.
template <int BITS, int NCH, int NPASS, int MAXK, bool SHARED_IN, bool USE_LDS, int WAVES, bool SPLIT>
__global__ __launch_bounds__(64 * WAVES) void k_down_combine(DownParams p) {
  constexpr int kThreads = 64 * WAVES;
  static_assert(!SPLIT || WAVES % 2 == 0, "waves pair up");
  // [K (+1)][I]: the SwiGLU outputs, staged once, each code chunk's columns
  // followed by kLdsPad unused floats
  extern __shared__ float hl[];
  constexpr int XSH = USE_LDS ? XS_LDSPAD : XS_F32;
  constexpr int NC = ChunkGeom<BITS>::kCols;
  const int wv = wave_uniform(threadIdx.x >> 6);
  const int wave = wave_uniform(SPLIT ? blockIdx.x * (WAVES / 2) + (wv >> 1) : blockIdx.x * WAVES + wv);
  const int half = SPLIT ? (wv & 1) : 0;
  const RowMap m = row_map<BITS>(p.I);
  const int row0 = wave * p.rows_per_wave;
  const bool active = row0 < p.H;
  // experts in order: the shared one (if here), then the routed ones
  constexpr int SIN = SHARED_IN ? 1 : 0;
  const int n_first = (p.K + SIN + 1) / 2;
  auto mine = [&](int slot) { return !SPLIT || ((slot < n_first) == (half == 0)); };

  // Loads in the order their data are needed (vmcnt counts in order): the
  // selection, the shared expert's rows (known before the selection), the
  // SwiGLU outputs for LDS, then the routed rows once the ids have arrived.
  // Only the LDS fill waits at the barrier; each expert's rows are consumed
  // as they arrive.
  int ids[MAXK];
  float wk[MAXK];
#pragma unroll
  for (int k = 0; k < MAXK; ++k) {
    ids[k] = k < p.K ? p.idx[k] : -2;
    wk[k] = k < p.K ? p.w[k] : 0.f;
  }
  DnTile<BITS, NCH, NPASS> ts;
  if constexpr (SHARED_IN) {
    if (mine(0)) down_load(ts, p.shared_rec, p.soff, p.H, m, row0);
  }
  const int lds_stride = (p.I / NC) * (NC + kLdsPad);  // floats per expert in LDS
  // float4 per thread held in registers (8192 values); the rest, if any, go
  // through a plain loop after the barrier's other loads
  constexpr int kHRegs = 2048 / kThreads;
  float4 hv[kHRegs];
  const int nh = (p.K + (SHARED_IN ? 1 : 0)) * p.I;
  const int nr = p.K * p.I;
  if constexpr (USE_LDS) {
    // branch-free: positions past the end load element 0 and are not stored
#pragma unroll
    for (int i = 0; i < kHRegs; ++i) {
      const int e0 = (i * kThreads + threadIdx.x) * 4;
      const int e = e0 < nh ? e0 : 0;
      const float *src = e < nr ? p.h_routed + e : p.h_shared + (e - nr);
      hv[i] = *reinterpret_cast<const float4 *>(src);
    }
  }
  DnTile<BITS, NCH, NPASS> t[MAXK];
#pragma unroll
  for (int k = 0; k < MAXK; ++k) {
    if (k < p.K && mine(k + SIN)) {  // wave-uniform
      ids[k] = wave_uniform(ids[k]);
      const bool v = ids[k] >= 0 && ids[k] < p.E;
      down_load(t[k], p.experts + (size_t)(v ? ids[k] : 0) * p.stride, p.off, p.H, m, row0);
    }
  }
  if constexpr (USE_LDS) {
    // expert of element e: (e + 0.5) / I rounded down, exact in fp32 here
    // (e < 2^17 and the quotient stays at least 0.5 / I from an integer)
    const float inv_i = 1.0f / (float)p.I;
    // (a code chunk's lanes are consecutive and agree on e < nh: I is a
    // multiple of the chunk width)
#pragma unroll
    for (int i = 0; i < kHRegs; ++i) {
      const int e = (i * kThreads + threadIdx.x) * 4;
      if (e < nh) {
        const int k = (int)(((float)e + 0.5f) * inv_i);
        lds_put_chunk4<BITS>(hl + k * lds_stride, e - k * p.I, hv[i]);
      }
    }
    for (int e = (kHRegs * kThreads + threadIdx.x) * 4; e < nh; e += kThreads * 4) {
      const float4 v = e < nr ? *reinterpret_cast<const float4 *>(p.h_routed + e)
                              : *reinterpret_cast<const float4 *>(p.h_shared + (e - nr));
      const int k = (int)(((float)e + 0.5f) * inv_i);
      lds_put_chunk4<BITS>(hl + k * lds_stride, e - k * p.I, v);
    }
    __syncthreads();
  }
  // (split pairs meet at a second barrier: their waves stay to the end; rows
  // past H are masked where they are loaded and stored)
  if (!SPLIT && !active) return;
  const int hstride = USE_LDS ? lds_stride : p.I;
  const float *hr = USE_LDS ? hl : p.h_routed;
  const float *hs = USE_LDS ? hl + (size_t)p.K * lds_stride : p.h_shared;

  float acc[NPASS];
#pragma unroll
  for (int i = 0; i < NPASS; ++i) acc[i] = 0.f;
  const float sig = p.sigma[0];
  if constexpr (SHARED_IN) {
    if (mine(0)) down_accumulate<BITS, NCH, NPASS, XSH>(hs, m, p.H, row0, true, sig, ts, acc);
  }
#pragma unroll
  for (int k = 0; k < MAXK; ++k) {
    if (k < p.K && mine(k + SIN)) {
      const bool v = ids[k] >= 0 && ids[k] < p.E;
      down_accumulate<BITS, NCH, NPASS, XSH>(hr + (size_t)k * hstride, m, p.H, row0, v, wk[k], t[k], acc);
    }
  }
  if constexpr (SPLIT) {
    __shared__ float part[WAVES / 2][NPASS][64];
    if (half) {
#pragma unroll
      for (int i = 0; i < NPASS; ++i) part[wv >> 1][i][lane_id()] = acc[i];
    }
    __syncthreads();
    if (half || !active) return;
#pragma unroll
    for (int i = 0; i < NPASS; ++i) acc[i] += part[wv >> 1][i][lane_id()];
  }
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
  // unreadable entries (see k_gateup) read routed record 0 and yield NaN
  const bool shared = id == kSharedId;
  const bool valid = shared ? (p.shared_ok != 0) : (id >= 0 && id < p.E);
  const bool from_shared = shared && valid;
  const uint8_t *rec = from_shared ? p.shared_rec : p.experts + (size_t)(valid && !shared ? id : 0) * p.stride;
  DnTile<BITS, NCH, NPASS> t;
  down_load(t, rec, from_shared ? p.soff : p.off, p.H, m, row0);
  float acc[NPASS];
#pragma unroll
  for (int i = 0; i < NPASS; ++i) acc[i] = 0.f;
  down_accumulate<BITS, NCH, NPASS, XS_F32>(p.h + (size_t)slot * p.I, m, p.H, row0, valid, 1.0f, t, acc);
#pragma unroll
  for (int i = 0; i < NPASS; ++i) {
    const float s = seg_sum(acc[i], m.lg);
    const int r = row0 + i * m.rpp + m.rip;
    if (m.li == 0 && r < p.H) p.y[(size_t)slot * p.H + r] = s;
  }
}

// ---------------------------------------------------------------------------
// expert tier: one wave takes the top-K of the token's logits, then gives
// each selected expert its cache slot.  The slot table (owner and last use
// of every slot) is copied to LDS, updated there expert by expert in the
// order of the selection, and the slots this token used are written back.
// A hit reads its slot; a miss takes the least recently used slot this token
// has not used (never-used slots first, the lowest index among equal uses),
// and the expert kernels read its record from host memory and write it into
// the slot as they go.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return ~wave_max_u32(~v); }

__global__ __launch_bounds__(64) void k_tier_route(TierRouteParams p) {
  __shared__ int32_t own[kMaxE];
  __shared__ uint32_t used[kMaxE];
  const int lane = lane_id();
  TierState *st = reinterpret_cast<TierState *>(p.state);
  int32_t *g_own = reinterpret_cast<int32_t *>(p.state + kTierOwnerOff);
  uint32_t *g_used = reinterpret_cast<uint32_t *>(g_own + p.n_slots);
  for (int j = lane; j < p.n_slots; j += 64) {
    own[j] = g_own[j];
    used[j] = g_used[j];
  }
  const uint32_t tick = st->tick + 1u;
  float v[kTopkNpl];
  topk_load(p.logits, p.E, v);
  int e;
  float w;
  topk_select(v, p.E, p.K, p.renorm, e, w);
  topk_store(e, w, p.K, p.idx, p.w);
  __syncthreads();
  int my_slot = -1, my_miss = 0;
#pragma unroll 1
  for (int k = 0; k < p.K; ++k) {
    const int ek = __builtin_amdgcn_readlane(e, k);
    int s = -1, miss = 0;
    if (ek >= 0) {  // uniform; a NaN logit can leave a selection empty
      int found = -1;
      for (int j = lane; j < p.n_slots; j += 64)
        if (own[j] == ek) found = j;
      const uint64_t b = __ballot(found >= 0);
      if (b) {
        s = __builtin_amdgcn_readlane(found, __builtin_ctzll(b));
      } else {
        uint32_t bu = 0xFFFFFFFFu, bj = 0xFFFFFFFFu;
        for (int j = lane; j < p.n_slots; j += 64)
          if (used[j] < tick && used[j] < bu) {  // ascending j: the first keeps ties
            bu = used[j];
            bj = (uint32_t)j;
          }
        const uint32_t mu = wave_min_u32(bu);
        s = (int)wave_min_u32(bu == mu ? bj : 0xFFFFFFFFu);
        miss = 1;
      }
      if (lane == 0) {
        own[s] = ek;
        used[s] = tick;
      }
      __syncthreads();
    }
    if (lane == k) {
      my_slot = s;
      my_miss = miss;
    }
  }
  if (lane < p.K) {
    p.slot[lane] = my_slot;
    const uint8_t *slot_rec = p.cache + (size_t)(my_slot >= 0 ? my_slot : 0) * p.stride;
    const uint8_t *host_rec = p.host_dev + (size_t)(e >= 0 ? e : 0) * p.stride;
    p.rec_src[lane] = reinterpret_cast<uint64_t>(my_miss ? host_rec : slot_rec);
    p.rec_fill[lane] = my_miss ? reinterpret_cast<uint64_t>(slot_rec) : 0ull;
  }
  for (int j = lane; j < p.n_slots; j += 64) {
    if (used[j] == tick) {
      g_own[j] = own[j];
      g_used[j] = tick;
    }
  }
  const int n_miss = __builtin_popcountll(__ballot(lane < p.K && my_miss));
  const int n_valid = __builtin_popcountll(__ballot(lane < p.K && my_slot >= 0));
  if (lane == 0) {
    st->tick = tick;
    st->hits += (unsigned long long)(n_valid - n_miss);
    st->misses += (unsigned long long)n_miss;
    st->bytes += (unsigned long long)n_miss * p.record_bytes;
  }
}

__global__ __launch_bounds__(kBlock) void k_tier_reset(uint8_t *state, int n_slots) {
  TierState *st = reinterpret_cast<TierState *>(state);
  int32_t *own = reinterpret_cast<int32_t *>(state + kTierOwnerOff);
  uint32_t *used = reinterpret_cast<uint32_t *>(own + n_slots);
  for (int j = threadIdx.x; j < n_slots; j += kBlock) {
    own[j] = -1;
    used[j] = 0u;
  }
  if (threadIdx.x == 0) {
    st->tick = 0u;
    st->pad[0] = 0u;
    st->hits = st->misses = st->bytes = 0ull;
  }
}

// ---------------------------------------------------------------------------
// token batches
// ---------------------------------------------------------------------------
// One workgroup: the top-K of every token (wave w takes tokens w, w + 4, ...),
// then a counting sort of the T*K (token, expert) pairs by expert id with the
// pair order kept inside an expert.  P = T*K <= 512 and the ranks are plain
// counts over the pairs, so the result does not depend on thread timing.
constexpr int kGroupBlock = 1024;  // one wave per token for up to 16 tokens at a time

__global__ __launch_bounds__(kGroupBlock) void k_route_group(RouteGroupParams p) {
  __shared__ int pe[kMaxTokens * kMaxK];
  __shared__ int pless[kMaxTokens * kMaxK];
  __shared__ unsigned char pfirst[kMaxTokens * kMaxK];
  __shared__ int n_first;
  const int wv = threadIdx.x >> 6, lane = lane_id();
  if (threadIdx.x == 0) n_first = 0;
  for (int t = wv; t < p.T; t += kGroupBlock / 64) {
    float v[kTopkNpl];
    topk_load(p.logits + (size_t)t * p.E, p.E, v);
    int e;
    float w;
    topk_select(v, p.E, p.K, p.renorm, e, w);
    topk_store(e, w, p.K, p.idx + (size_t)t * p.K, p.w + (size_t)t * p.K);
    if (lane < p.K) pe[t * p.K + lane] = e;
  }
  __syncthreads();
  const int P = p.T * p.K;
  int mine = 0;
  for (int q = threadIdx.x; q < P; q += kGroupBlock) {
    const int e = pe[q];
    int less = 0, before = 0;
    for (int r = 0; r < P; ++r) {
      const int f = pe[r];
      less += f < e;
      before += (r < q) & (f == e);
    }
    p.g_pair[less + before] = q;
    pless[q] = less;
    pfirst[q] = before == 0;
    mine += before == 0;
  }
  atomicAdd(&n_first, mine);
  __syncthreads();
  for (int q = threadIdx.x; q < P; q += kGroupBlock) {
    if (!pfirst[q]) continue;
    const int e = pe[q];
    int g = 0;
    for (int r = 0; r < P; ++r) g += pfirst[r] & (pe[r] < e);
    p.g_expert[g] = e;
    p.g_start[g] = pless[q];
  }
  if (threadIdx.x == 0) {
    p.g_count[0] = n_first;
    p.g_start[n_first] = P;
  }
}

// the group of a work item: its expert (or the shared one) and its tokens;
// lane j < n holds the j-th (pair, token) of the group
struct GroupRef {
  int id, n, pair, tok;
  bool shared;
};

// Work items, in order: the shared expert's (its T tokens in shared_split
// ranges, each range over every row tile: it holds the most work, so it
// starts first and no item carries every token), then the row tiles of the
// routed groups in expert order.  Returns the item's group and row tile.
__device__ __forceinline__ int n_work_items(const GroupedParams &p, int U) {
  return ((p.do_shared ? p.shared_split : 0) + U) * p.tiles;
}

__device__ __forceinline__ GroupRef item_ref(const GroupedParams &p, int item, int U, int &tile) {
  GroupRef r;
  const int lane = lane_id();
  const int n_sh = p.do_shared ? p.shared_split * p.tiles : 0;
  if (item < n_sh) {
    const int part = item / p.tiles;
    tile = item - part * p.tiles;
    const int per = (p.T + p.shared_split - 1) / p.shared_split;
    const int t0 = part * per;
    r.shared = true;
    r.id = kSharedId;
    r.n = p.T - t0 < per ? p.T - t0 : per;
    r.pair = t0 + lane;
    r.tok = t0 + lane;
  } else {
    const int q = item - n_sh;
    const int g = q / p.tiles;
    tile = q - g * p.tiles;
    r.shared = false;
    r.id = wave_uniform(p.g_expert[g]);
    const int s0 = wave_uniform(p.g_start[g]);
    r.n = wave_uniform(p.g_start[g + 1]) - s0;
    r.pair = lane < r.n ? p.g_pair[s0 + lane] : 0;
    r.tok = r.pair / p.K;
  }
  return r;
}

// ---- staged activations in LDS, shared by the workgroup's four waves ----
// A chunk's LDS slot: its stage's words rounded up to a multiple of 4 and, if
// that count of 16-byte units is even, one unit more, so that lanes reading
// consecutive chunks start in different bank groups.
template <typename Stage>
__host__ __device__ constexpr int lds_chunk_words() {
  constexpr int n = ((int)(sizeof(Stage) / 4) + 3) / 4 * 4;
  return (n / 4) % 2 == 0 ? n + 4 : n;
}

template <int BITS>
__device__ __forceinline__ void lds_store(uint32_t *d, const XStage<BITS, false> &s) {
  constexpr int NP = ChunkGeom<BITS>::kPairs;
#pragma unroll
  for (int i = 0; i < NP / 4; ++i)
    reinterpret_cast<uint4 *>(d)[i] = make_uint4(s.p[4 * i], s.p[4 * i + 1], s.p[4 * i + 2], s.p[4 * i + 3]);
  *reinterpret_cast<float2 *>(d + NP) = make_float2(s.off, s.xs);
}
template <int BITS>
__device__ __forceinline__ void lds_load(const uint32_t *d, XStage<BITS, false> &s) {
  constexpr int NP = ChunkGeom<BITS>::kPairs;
#pragma unroll
  for (int i = 0; i < NP / 4; ++i) {
    const uint4 u = reinterpret_cast<const uint4 *>(d)[i];
    s.p[4 * i] = u.x;
    s.p[4 * i + 1] = u.y;
    s.p[4 * i + 2] = u.z;
    s.p[4 * i + 3] = u.w;
  }
  const float2 t = *reinterpret_cast<const float2 *>(d + NP);
  s.off = t.x;
  s.xs = t.y;
}
template <int BITS>
__device__ __forceinline__ void lds_store(uint32_t *d, const XStage<BITS, true> &s) {
  constexpr int NC = ChunkGeom<BITS>::kCols;
#pragma unroll
  for (int i = 0; i < NC / 4; ++i)
    reinterpret_cast<float4 *>(d)[i] = make_float4(s.v[4 * i], s.v[4 * i + 1], s.v[4 * i + 2], s.v[4 * i + 3]);
  reinterpret_cast<float *>(d)[NC] = s.xs;
}
template <int BITS>
__device__ __forceinline__ void lds_load(const uint32_t *d, XStage<BITS, true> &s) {
  constexpr int NC = ChunkGeom<BITS>::kCols;
#pragma unroll
  for (int i = 0; i < NC / 4; ++i) {
    const float4 u = reinterpret_cast<const float4 *>(d)[i];
    s.v[4 * i] = u.x;
    s.v[4 * i + 1] = u.y;
    s.v[4 * i + 2] = u.z;
    s.v[4 * i + 3] = u.w;
  }
  s.xs = reinterpret_cast<const float *>(d)[NC];
}

// stage chunk c of token tok's x (from the staged buffer when there is one)
template <int BITS, int XS>
__device__ __forceinline__ XStage<BITS, XS != XS_BF16> group_stage_chunk(const GroupedParams &p,
                                                                         int tok, int c) {
  if constexpr (XS == XS_BF16) {
    if (p.xs_pairs)
      return read_stage<BITS>(p.xs_pairs + (size_t)tok * p.xs_pair_stride,
                              p.xs_sums + (size_t)tok * p.xs_sum_stride, c);
    return make_stage<BITS, XS>(static_cast<const uint16_t *>(p.x) + (size_t)tok * p.H, nullptr, c);
  } else {
    return make_stage<BITS, XS>(static_cast<const float *>(p.x) + (size_t)tok * p.H, nullptr, c);
  }
}

constexpr int kGroupTB = 4;  // tokens that share one unpacking of a code chunk

// Work items are (group, block tile): the workgroup's four waves take
// consecutive row tiles of one expert group, so the tokens' activations are
// staged into LDS once per workgroup, tok_batch tokens at a time, and read
// there by all four waves.
template <int BITS, int NCH, int NPASS, int XS>
__global__ __launch_bounds__(kBlock) void k_gateup_grouped(GroupedParams p) {
  extern __shared__ uint32_t lds_x[];
  constexpr bool XF32 = XS != XS_BF16;
  using Stage = XStage<BITS, XF32>;
  constexpr int CS = lds_chunk_words<Stage>();
  const int wv = wave_uniform(threadIdx.x >> 6);
  const int U = p.do_routed ? wave_uniform(p.g_count[0]) : 0;
  const int n_items = n_work_items(p, U);
  const RowMap m = row_map<BITS>(p.H);
  const int cpr = m.cpr;
  const uint32_t magic = opaque(kMagic16);
  // the next item's weight rows are requested while this item's tokens are
  // worked through
  GUTile<BITS, NCH, NPASS> next;
  GroupRef ngr;
  int nrow0 = 0;
  auto fetch = [&](int item, GUTile<BITS, NCH, NPASS> &t, GroupRef &r, int &row0) {
    int tile;
    r = item_ref(p, item < n_items ? item : 0, U, tile);
    row0 = (tile * 4 + wv) * p.rows_per_wave;
    const bool v = r.shared ? true : (r.id >= 0 && r.id < p.E);
    const uint8_t *rec = r.shared ? p.shared_rec : p.experts + (size_t)(v ? r.id : 0) * p.stride;
    gu_load(t, rec, r.shared ? p.soff : p.off, m, p.I, row0);
  };
  if (blockIdx.x < n_items) fetch(blockIdx.x, next, ngr, nrow0);
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const GUTile<BITS, NCH, NPASS> tile = next;
    const GroupRef gr = ngr;
    const int row0 = nrow0;
    const bool valid = gr.shared ? true : (gr.id >= 0 && gr.id < p.E);
    for (int i0 = 0; i0 < gr.n; i0 += p.tok_batch) {
      const int nb = gr.n - i0 < p.tok_batch ? gr.n - i0 : p.tok_batch;
      __syncthreads();  // the previous batch has been read
      // the trip count is the same for every thread, so every lane is active
      // at the shuffle (a lane cannot read an inactive lane's register)
      for (int base = 0; base < nb * cpr; base += kBlock) {
        const int idx = base + threadIdx.x;
        const int b = idx / cpr, c = idx - b * cpr;
        const int tok = __shfl(gr.tok, (i0 + b) & 63, 64);
        if (idx < nb * cpr)
          lds_store<BITS>(lds_x + (size_t)(b * cpr + c) * CS, group_stage_chunk<BITS, XS>(p, tok, c));
      }
      __syncthreads();
      // the next item's weight rows are requested once this item's first
      // activations are staged: loads complete in order, so requested
      // earlier they would hold up the staging
      if (i0 == 0 && item + (int)gridDim.x < n_items) fetch(item + gridDim.x, next, ngr, nrow0);
      if constexpr (!XF32) {
        // bf16 x: each code chunk is made into bf16 pairs once for up to
        // kGroupTB tokens, which then take only the dot products (the same
        // operations in the same order as gu_compute, token by token)
        for (int b0 = 0; b0 < nb; b0 += kGroupTB) {
          const int nt = nb - b0 < kGroupTB ? nb - b0 : kGroupTB;  // uniform
          float a[kGroupTB][NPASS], u[kGroupTB][NPASS];
#pragma unroll
          for (int t = 0; t < kGroupTB; ++t)
#pragma unroll
            for (int q = 0; q < NPASS; ++q) a[t][q] = u[t][q] = 0.f;
#pragma unroll
          for (int q = 0; q < NPASS; ++q) {
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
              const bool in = in_tile(m, p.I, row0, q, j);
              const uint32_t gsw = in ? tile.gs[q][j] : 0u, usw = in ? tile.us[q][j] : 0u;
              uint32_t gpr[ChunkGeom<BITS>::kPairs], upr[ChunkGeom<BITS>::kPairs];
              chunk_pairs<BITS>(tile.gq[q][j], magic, gpr);
              chunk_pairs<BITS>(tile.uq[q][j], magic, upr);
              const int c0 = m.li + (j << m.lg);
              const int cc = c0 < cpr ? c0 : 0;
#pragma unroll
              for (int t = 0; t < kGroupTB; ++t) {
                if (t < nt) {  // uniform
                  Stage xs;
                  lds_load<BITS>(lds_x + (size_t)((b0 + t) * cpr + cc) * CS, xs);
                  float da = -xs.off, du = -xs.off;
#pragma unroll
                  for (int i = 0; i < ChunkGeom<BITS>::kPairs; ++i) {
                    da = dot2bf(gpr[i], xs.p[i], da);
                    du = dot2bf(upr[i], xs.p[i], du);
                  }
                  a[t][q] = fmaf(bf_lo(gsw), da, fmaf(bf_hi(gsw), xs.xs, a[t][q]));
                  u[t][q] = fmaf(bf_lo(usw), du, fmaf(bf_hi(usw), xs.xs, u[t][q]));
                }
              }
            }
          }
#pragma unroll
          for (int t = 0; t < kGroupTB; ++t) {
            if (t < nt) {  // uniform
              const int pair = __builtin_amdgcn_readlane(gr.pair, i0 + b0 + t);
              const int tok = __builtin_amdgcn_readlane(gr.tok, i0 + b0 + t);
              float *hout = gr.shared ? p.h_shared + (size_t)tok * p.I : p.h_routed + (size_t)pair * p.I;
#pragma unroll
              for (int q = 0; q < NPASS; ++q) {
                const float sa = seg_sum(a[t][q], m.lg);
                const float su = seg_sum(u[t][q], m.lg);
                const int r = row0 + q * m.rpp + m.rip;
                if (m.li == 0 && r < p.I) hout[r] = valid ? silu_mul(sa, su) : __builtin_nanf("");
              }
            }
          }
        }
      } else {
        for (int b = 0; b < nb; ++b) {
          Stage xs[NCH];
#pragma unroll
          for (int j = 0; j < NCH; ++j) {
            const int c0 = m.li + (j << m.lg);
            lds_load<BITS>(lds_x + (size_t)(b * cpr + (c0 < cpr ? c0 : 0)) * CS, xs[j]);
          }
          const int pair = __builtin_amdgcn_readlane(gr.pair, i0 + b);
          const int tok = __builtin_amdgcn_readlane(gr.tok, i0 + b);
          float *hout = gr.shared ? p.h_shared + (size_t)tok * p.I : p.h_routed + (size_t)pair * p.I;
          gu_compute(tile, xs, m, p.I, row0, valid, hout);
        }
      }
    }
  }
}

// down projection over the groups; the SwiGLU outputs of a batch of tokens
// go to LDS (padded per code chunk) once per workgroup
template <int BITS, int NCH, int NPASS>
__global__ __launch_bounds__(kBlock) void k_down_grouped(GroupedParams p) {
  extern __shared__ float lds_h[];
  constexpr int NC = ChunkGeom<BITS>::kCols;
  constexpr int PC = NC + kLdsPad;
  const int wv = wave_uniform(threadIdx.x >> 6);
  const int U = p.do_routed ? wave_uniform(p.g_count[0]) : 0;
  const int n_items = n_work_items(p, U);
  const RowMap m = row_map<BITS>(p.I);
  const int tok_floats = (p.I / NC) * PC;
  DnTile<BITS, NCH, NPASS> next;
  GroupRef ngr;
  int nrow0 = 0;
  auto fetch = [&](int item, DnTile<BITS, NCH, NPASS> &t, GroupRef &r, int &row0) {
    int tile;
    r = item_ref(p, item < n_items ? item : 0, U, tile);
    row0 = (tile * 4 + wv) * p.rows_per_wave;
    const bool v = r.shared ? true : (r.id >= 0 && r.id < p.E);
    const uint8_t *rec = r.shared ? p.shared_rec : p.experts + (size_t)(v ? r.id : 0) * p.stride;
    down_load(t, rec, r.shared ? p.soff : p.off, p.H, m, row0);
  };
  if (blockIdx.x < n_items) fetch(blockIdx.x, next, ngr, nrow0);
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const DnTile<BITS, NCH, NPASS> tile = next;
    const GroupRef gr = ngr;
    const int row0 = nrow0;
    const bool valid = gr.shared ? true : (gr.id >= 0 && gr.id < p.E);
    for (int i0 = 0; i0 < gr.n; i0 += p.tok_batch) {
      const int nb = gr.n - i0 < p.tok_batch ? gr.n - i0 : p.tok_batch;
      __syncthreads();  // the previous batch has been read
      for (int b = 0; b < nb; ++b) {
        const int pair = __builtin_amdgcn_readlane(gr.pair, i0 + b);
        const int tok = __builtin_amdgcn_readlane(gr.tok, i0 + b);
        const float *hin = gr.shared ? p.h_shared + (size_t)tok * p.I : p.h_routed + (size_t)pair * p.I;
        for (int col = threadIdx.x * 4; col < p.I; col += kBlock * 4)
          lds_put_chunk4<BITS>(lds_h + b * tok_floats, col, *reinterpret_cast<const float4 *>(hin + col));
      }
      __syncthreads();
      // the next item's rows are requested once this item's first inputs are
      // staged (loads complete in order)
      if (i0 == 0 && item + (int)gridDim.x < n_items) fetch(item + gridDim.x, next, ngr, nrow0);
      for (int b = 0; b < nb; ++b) {
        const int pair = __builtin_amdgcn_readlane(gr.pair, i0 + b);
        const int tok = __builtin_amdgcn_readlane(gr.tok, i0 + b);
        float *yout = gr.shared ? p.y_shared + (size_t)tok * p.H : p.y_routed + (size_t)pair * p.H;
        XStage<BITS, true> xs[NCH];
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
          const int c = m.li + (j << m.lg);
          xs[j] = make_stage<BITS, XS_LDSPAD>(nullptr, lds_h + b * tok_floats, c < m.cpr ? c : 0);
        }
        float acc[NPASS];
#pragma unroll
        for (int k = 0; k < NPASS; ++k) acc[k] = 0.f;
        down_accumulate_staged<BITS, NCH, NPASS>(xs, m, p.H, row0, valid, 1.0f, tile, acc);
#pragma unroll
        for (int k = 0; k < NPASS; ++k) {
          const float sum = seg_sum(acc[k], m.lg);
          const int r = row0 + k * m.rpp + m.rip;
          if (m.li == 0 && r < p.H) yout[r] = sum;
        }
      }
    }
  }
}

__global__ __launch_bounds__(kBlock) void k_combine_tokens(CombineTokensParams p) {
  const int o = blockIdx.x * kBlock + threadIdx.x;
  const int t = blockIdx.y;
  if (o >= p.H) return;
  float acc = p.h_res[(size_t)t * p.H + o];
  for (int k = 0; k < p.K; ++k)
    acc = fmaf(p.w[t * p.K + k], p.y_routed[(size_t)(t * p.K + k) * p.H + o], acc);
  acc = fmaf(p.sigma[t], p.y_shared[(size_t)t * p.H + o], acc);
  p.out[(size_t)t * p.H + o] = acc;
}

// ---------------------------------------------------------------------------
// launch shapes
// ---------------------------------------------------------------------------

// Passes per wave (rows per wave = passes * rows per pass) of each kernel.
// MOE_TUNE="gu=<p>,dn=<p>,sh=<p>" (p = 1, 2 or 4) overrides the defaults.
struct Tune {
  int gu = 0, dn = 0, sh = 0;
};
static const Tune &tune() {
  static const Tune t = [] {
    Tune r;
    const char *e = getenv("MOE_TUNE");
    if (!e) return r;
    for (const char *s = e; *s;) {
      int v = 0;
      if (sscanf(s, "gu=%d", &v) == 1) r.gu = v;
      else if (sscanf(s, "dn=%d", &v) == 1) r.dn = v;
      else if (sscanf(s, "sh=%d", &v) == 1) r.sh = v;
      while (*s && *s != ',') ++s;
      if (*s == ',') ++s;
    }
    return r;
  }();
  return t;
}
static int pick_pass(int tuned, int dflt) {
  return (tuned == 1 || tuned == 2 || tuned == 4) ? tuned : dflt;
}

// instantiated (NCH, NPASS) pairs: NCH 2 with at most two passes, NCH 4
// (rows wider than 2048 codes per 64 lanes) with one
#define MOE_DISPATCH(nch, npass, ...)                                                    \
  do {                                                                                   \
    if (nch == 1 && npass == 1) { constexpr int NCH_ = 1, NP_ = 1; __VA_ARGS__; }        \
    else if (nch == 1 && npass == 2) { constexpr int NCH_ = 1, NP_ = 2; __VA_ARGS__; }   \
    else if (nch == 1) { constexpr int NCH_ = 1, NP_ = 4; __VA_ARGS__; }                 \
    else if (nch == 2 && npass == 1) { constexpr int NCH_ = 2, NP_ = 1; __VA_ARGS__; }   \
    else if (nch == 2) { constexpr int NCH_ = 2, NP_ = 2; __VA_ARGS__; }                 \
    else { constexpr int NCH_ = 4, NP_ = 1; __VA_ARGS__; }                              \
  } while (0)


size_t xstage_pair_bytes(int cols, int bits) {
  return (size_t)(cols * bits / 128) * (64 / bits) * 4;
}
size_t xstage_sum_bytes(int cols, int bits) { return (size_t)(cols * bits / 128) * 8; }

hipError_t launch_head(const HeadParams &p0, hipStream_t s) {
  HeadParams p = p0;
  const int bs = p.n_shared_waves > 0 ? p.bits_shared : 0;
  const int nch = bs ? nch_for(p.H, bs) : 1;
  const int npass = bs ? clamp_pass(nch, pick_pass(tune().sh, 2)) : 1;
  if (bs) {  // size the shared-expert part of the grid
    p.shared_rows_per_wave = npass * rpp_for(p.H, bs);
    p.n_shared_waves = (p.I + p.shared_rows_per_wave - 1) / p.shared_rows_per_wave;
  }
  const int units = p.T * (p.E + 1) + p.T;  // rows of every token, then one x stager per token
  // two waves per workgroup unless the norm prologue or the shared expert's
  // rows run here (q4 layer: 20.64 -> 20.50 us per layer)
  const int W = (bs == 0 && p.xsrc != XS_NORM) ? 2 : 4;
  p.n_router_blocks = (units + W - 1) / W;
  const int nsb = bs ? (p.n_shared_waves + 3) / 4 : 0;
  const dim3 grid(p.n_router_blocks + nsb);
  const size_t lds = p.xsrc == XS_NORM ? (size_t)p.H * sizeof(float) : 0;
#define MOE_HEAD(XS)                                                                             \
  if (bs == 4) {                                                                                 \
    MOE_DISPATCH(nch, npass,                                                                     \
                 MOE_LAUNCH((k_head<XS, 4, NCH_, NP_>), grid, dim3(kBlock), lds, s, p)); \
  } else if (bs == 2) {                                                                          \
    MOE_DISPATCH(nch, npass,                                                                     \
                 MOE_LAUNCH((k_head<XS, 2, NCH_, NP_>), grid, dim3(kBlock), lds, s, p)); \
  } else {                                                                                       \
    MOE_LAUNCH((k_head<XS, 0, 1, 1>), grid, dim3(64 * W), lds, s, p);                    \
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
  MOE_LAUNCH(k_topk, dim3(p.T), dim3(64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gateup(const GateUpParams &p0, hipStream_t s) {
  GateUpParams p = p0;
  const int nch = nch_for(p.H, p.bits);
  const int rpp = rpp_for(p.H, p.bits);
  const int npass = clamp_pass(nch, pick_pass(tune().gu, rpp >= 2 ? 1 : 2));
  p.rows_per_wave = npass * rpp;
  p.waves_per_expert = (p.I + p.rows_per_wave - 1) / p.rows_per_wave;
  p.n_shared_blocks = p.with_shared ? (p.waves_per_expert + 3) / 4 : 0;
  const int waves = p.waves_per_expert * p.n;
  p.n_copy_blocks = 0;
  if (p.rec_fill) {  // the tier's down-section copies: about 36 KiB per workgroup
    const size_t bytes = (size_t)p.H * p.I * p.bits / 8 + (size_t)p.H * (p.I / kGroup) * 4;
    p.copy_blocks_per_entry = (int)((bytes + 36863) / 36864);
    p.n_copy_blocks = p.copy_blocks_per_entry * p.n;
  }
  const dim3 grid(p.n_shared_blocks + (waves + 3) / 4 + p.n_copy_blocks);
#define MOE_GU(BITS, XS)                                                                        \
  do {                                                                                           \
    if constexpr (gateup_x_in_lds(BITS, XS)) {                                                   \
      const size_t lds = (size_t)(p.H * BITS / 128) * XLds<BITS, XS != XS_BF16>::kWords * 4;    \
      MOE_DISPATCH(nch, npass, MOE_LAUNCH((k_gateup_xl<BITS, NCH_, NP_, XS>), grid,            \
                                          dim3(kBlock), lds, s, p));                             \
    } else {                                                                                     \
      MOE_DISPATCH(nch, npass, MOE_LAUNCH((k_gateup<BITS, NCH_, NP_, XS>), grid, dim3(kBlock),  \
                                          0, s, p));                                             \
    }                                                                                            \
  } while (0)
  if (p.bits == 4) {
    if (p.xsrc == XS_BF16) { MOE_GU(4, XS_BF16); } else { MOE_GU(4, XS_F32); }
  } else {
    if (p.xsrc == XS_BF16) { MOE_GU(2, XS_BF16); } else { MOE_GU(2, XS_F32); }
  }
#undef MOE_GU
  return hipGetLastError();
}

hipError_t launch_down(const DownParams &p0, hipStream_t s) {
  DownParams p = p0;
  const int bits = p.bits_r;
  const int nch = nch_for(p.I, bits);
  const int rpp = rpp_for(p.I, bits);
  const int npass = clamp_pass(nch, pick_pass(tune().dn, rpp >= 2 ? 1 : 2));
  p.rows_per_wave = npass * rpp;
  if (p.combine) {
    const bool shared_in = p.h_shared != nullptr;
    const int waves = (p.H + p.rows_per_wave - 1) / p.rows_per_wave;
    const bool k4 = p.K <= 4;
    // the SwiGLU outputs go through LDS (padded per code chunk) when they fit
    // in 64 KiB
    const int nc = 128 / bits;
    const size_t hbytes = (size_t)(p.K + (shared_in ? 1 : 0)) * (p.I / nc) * (nc + kLdsPad) * sizeof(float);
    const bool use_lds = hbytes <= 65536;
    const size_t lds = use_lds ? hbytes : 0;
    // eight-wave workgroups when there are enough waves for one per CU (q4
    // layer: 20.85 against 21.15 us; with 1024 waves, half the CUs would idle)
    const bool eight = use_lds && waves >= 8 * kCUs;
    // otherwise (fewer rows) two waves share each set of rows, splitting the
    // experts, so that the grid still has waves to hide latency with
    const bool split = use_lds && !eight;
    const dim3 grid(eight ? (waves + 7) / 8 : (split ? (waves + 1) / 2 : (waves + 3) / 4));
#define MOE_DC(BITS, MAXK, SIN)                                                                       \
  do {                                                                                                \
    if (eight)                                                                                        \
      MOE_DISPATCH(nch, npass, MOE_LAUNCH((k_down_combine<BITS, NCH_, NP_, MAXK, SIN, true, 8, false>), \
                                          grid, dim3(512), lds, s, p));                               \
    else if (split)                                                                                   \
      MOE_DISPATCH(nch, npass, MOE_LAUNCH((k_down_combine<BITS, NCH_, NP_, MAXK, SIN, true, 4, true>), \
                                          grid, dim3(kBlock), lds, s, p));                            \
    else                                                                                              \
      MOE_DISPATCH(nch, npass, MOE_LAUNCH((k_down_combine<BITS, NCH_, NP_, MAXK, SIN, false, 4, false>), \
                                          grid, dim3(kBlock), 0, s, p));                              \
  } while (0)
    if (bits == 4) {
      if (shared_in) { if (k4) MOE_DC(4, 4, true); else MOE_DC(4, 8, true); }
      else { if (k4) MOE_DC(4, 4, false); else MOE_DC(4, 8, false); }
    } else {
      if (shared_in) { if (k4) MOE_DC(2, 4, true); else MOE_DC(2, 8, true); }
      else { if (k4) MOE_DC(2, 4, false); else MOE_DC(2, 8, false); }
    }
#undef MOE_DC
  } else {
    p.waves_per_expert = (p.H + p.rows_per_wave - 1) / p.rows_per_wave;
    const int waves = p.waves_per_expert * p.n;
    const dim3 grid((waves + 3) / 4);
#define MOE_DY(BITS)                                                                           \
  MOE_DISPATCH(nch, npass, MOE_LAUNCH((k_down_y<BITS, NCH_, NP_>), grid, dim3(kBlock),  \
                                              0, s, p))
    if (bits == 4) { MOE_DY(4); } else { MOE_DY(2); }
#undef MOE_DY
  }
  return hipGetLastError();
}

hipError_t launch_tier_route(const TierRouteParams &p, hipStream_t s) {
  MOE_LAUNCH(k_tier_route, dim3(1), dim3(64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_tier_reset(uint8_t *state, int n_slots, hipStream_t s) {
  MOE_LAUNCH(k_tier_reset, dim3(1), dim3(kBlock), 0, s, state, n_slots);
  return hipGetLastError();
}

hipError_t launch_route_group(const RouteGroupParams &p, hipStream_t s) {
  MOE_LAUNCH(k_route_group, dim3(1), dim3(kGroupBlock), 0, s, p);
  return hipGetLastError();
}

// block tiles of four waves; a grid of at most 768 workgroups (three per CU,
// what the kernels' register use lets a CU hold) takes the work items in a
// strided loop; LDS holds up to 48 KiB of staged activations
#define MOE_DISPATCH_G(nch, npass, ...)                                                  \
  do {                                                                                   \
    if (nch == 1 && npass == 1) { constexpr int NCH_ = 1, NP_ = 1; __VA_ARGS__; }        \
    else if (nch == 1 && npass == 2) { constexpr int NCH_ = 1, NP_ = 2; __VA_ARGS__; }   \
    else if (nch == 1) { constexpr int NCH_ = 1, NP_ = 4; __VA_ARGS__; }                 \
    else if (nch == 2 && npass == 1) { constexpr int NCH_ = 2, NP_ = 1; __VA_ARGS__; }   \
    else if (nch == 2 && npass <= 2) { constexpr int NCH_ = 2, NP_ = 2; __VA_ARGS__; }   \
    else if (nch == 2) { constexpr int NCH_ = 2, NP_ = 4; __VA_ARGS__; }                 \
    else { constexpr int NCH_ = 4, NP_ = 1; __VA_ARGS__; }                              \
  } while (0)

static constexpr size_t kGroupedLds = 48 * 1024;

// the shared expert's tokens in at most four ranges
static void set_shared_split(GroupedParams &p) {
  const int per = (p.T + 3) / 4;
  p.shared_split = (p.T + per - 1) / per;
}

static dim3 grouped_grid(const GroupedParams &p, long cap) {
  const int routed = p.do_routed ? (p.T * p.K < p.E ? p.T * p.K : p.E) : 0;
  long blocks = (long)(routed + (p.do_shared ? p.shared_split : 0)) * p.tiles;
  if (blocks > cap) blocks = cap;
  return dim3((unsigned)(blocks < 1 ? 1 : blocks));
}

static int tok_batch_for(size_t per_token, int T) {
  long n = (long)(kGroupedLds / per_token);
  if (n < 1) n = 1;
  return (int)(n < T ? n : T);
}

hipError_t launch_gateup_grouped(const GroupedParams &p0, hipStream_t s) {
  GroupedParams p = p0;
  const int nch = nch_for(p.H, p.bits);
  const int rpp = rpp_for(p.H, p.bits);
  // one pass of rows per wave: the lighter waves let three workgroups share
  // a CU (q4_batch16: 71 us for gate/up, against 76 us with two passes and
  // two workgroups per CU)
  const int npass = 1;
  p.rows_per_wave = npass * rpp;
  p.tiles = (p.I + 4 * p.rows_per_wave - 1) / (4 * p.rows_per_wave);
  set_shared_split(p);
  const dim3 grid = grouped_grid(p, 768);
  const int cpr = p.H * p.bits / 128;
#define MOE_GG(BITS, XS)                                                                       \
  do {                                                                                         \
    const size_t per_tok = (size_t)cpr * lds_chunk_words<XStage<BITS, XS != XS_BF16>>() * 4;   \
    p.tok_batch = tok_batch_for(per_tok, p.T);                                                 \
    const size_t lds = per_tok * p.tok_batch;                                                  \
    MOE_DISPATCH_G(nch, npass, MOE_LAUNCH((k_gateup_grouped<BITS, NCH_, NP_, XS>), grid,        \
                                          dim3(kBlock), lds, s, p));                           \
  } while (0)
  if (p.bits == 4) {
    if (p.xsrc == XS_BF16) { MOE_GG(4, XS_BF16); } else { MOE_GG(4, XS_F32); }
  } else {
    if (p.xsrc == XS_BF16) { MOE_GG(2, XS_BF16); } else { MOE_GG(2, XS_F32); }
  }
#undef MOE_GG
  return hipGetLastError();
}

hipError_t launch_down_grouped(const GroupedParams &p0, hipStream_t s) {
  GroupedParams p = p0;
  const int nch = nch_for(p.I, p.bits);
  const int rpp = rpp_for(p.I, p.bits);
  const int npass = nch >= 4 ? 1 : (rpp >= 8 ? 1 : (rpp >= 4 ? 2 : 4));
  p.rows_per_wave = npass * rpp;
  p.tiles = (p.H + 4 * p.rows_per_wave - 1) / (4 * p.rows_per_wave);
  set_shared_split(p);
  const dim3 grid = grouped_grid(p, 768);
  const int nc = 128 / p.bits;
  const size_t per_tok = (size_t)(p.I / nc) * (nc + kLdsPad) * 4;
  p.tok_batch = tok_batch_for(per_tok, p.T);
  const size_t lds = per_tok * p.tok_batch;
  if (p.bits == 4) {
    MOE_DISPATCH_G(nch, npass, MOE_LAUNCH((k_down_grouped<4, NCH_, NP_>), grid, dim3(kBlock), lds, s, p));
  } else {
    MOE_DISPATCH_G(nch, npass, MOE_LAUNCH((k_down_grouped<2, NCH_, NP_>), grid, dim3(kBlock), lds, s, p));
  }
  return hipGetLastError();
}

hipError_t launch_combine_tokens(const CombineTokensParams &p, hipStream_t s) {
  MOE_LAUNCH(k_combine_tokens, dim3((p.H + kBlock - 1) / kBlock, p.T), dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe_impl
