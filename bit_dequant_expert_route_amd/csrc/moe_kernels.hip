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
#include "moe_launch.h"

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
  // The router blocks take (row, token) units, the T tokens of a row
  // consecutive, then one x stager per token.  With several tokens the
  // blocks are dealt to the 8 XCDs in contiguous ranges (block b takes
  // position (b mod 8) (n / 8) + b / 8), so that a router row's tokens run in
  // one XCD and its bytes come into that XCD's L2 once (16 tokens: 35.9 MB
  // fetched per launch for the 4.2 MB router before).  One token keeps the
  // plain order.
  const int nb = p.n_router_blocks;
  const int pos = (p.T > 1 && nb % 8 == 0) ? (blk % 8) * (nb / 8) + blk / 8 : blk;
  const int unit = pos * wpb + wv;
  const int rows = p.E + 1;
  // the stack path normalises x in every workgroup: the router row is
  // requested first so that its latency overlaps the normalisation
  RowPre pre{};
  bool have_pre = false;
  // the dots of the rows are taken with h + u and scaled by the norm's
  // reciprocal when only dots read x here (no shared expert's rows)
  float rscale = 1.0f;
  if constexpr (XS == XS_NORM) {
    const int row = unit / p.T;
    if (blk < p.n_router_blocks && unit < p.T * rows && row < p.E) {
      const size_t esz = p.router_dtype == 1 ? 2 : 4;
      pre = row_prefetch(static_cast<const uint8_t *>(p.router) + (size_t)row * p.H * esz,
                         p.router_dtype, p.H);
      have_pre = true;
    }
    if constexpr (BITS_S == 0) rscale = norm_prologue_scaled(p, xl);
    else norm_prologue(p, xl);
  }
  if (blk < p.n_router_blocks) {
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
    const int row = unit / p.T, t = unit - row * p.T;
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
// one workgroup per token, the selection split over its four waves (as in
// the gate/up kernel: each wave selects over a quarter of the experts, then
// one wave merges the 4 K candidates)
__global__ __launch_bounds__(kBlock) void k_topk(TopkParams p) {
  __shared__ TopkShare tsh;
  static_assert(kBlock / 64 == 4, "the selection is split over four waves");
  const int t = blockIdx.x;
  const int wv = wave_uniform(threadIdx.x >> 6);
  const float *lg = p.logits + (size_t)t * p.E;
  float lv[4];
  if (topk_npl(p.E) == 2) {
    topk_part_load<2>(lg, p.E, wv, lv);
    topk_part_select<2>(lv, p.E, p.K, p.renorm, wv, tsh);
  } else {
    topk_part_load<4>(lg, p.E, wv, lv);
    topk_part_select<4>(lv, p.E, p.K, p.renorm, wv, tsh);
  }
  __syncthreads();
  if (wv != 0) return;
  int sel_e = -2;
  uint32_t sel_key = 0, top_key = 0;
  topk_merge(tsh, p.E, p.K, sel_e, sel_key, top_key);
  topk_store(sel_e, topk_merge_weight(tsh, p.K, p.renorm, sel_e, sel_key, top_key), p.K,
             p.idx + (size_t)t * p.K, p.w + (size_t)t * p.K);
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
// K2 with x staged once per workgroup in LDS (XLds): each thread loads a slice
// of x before the one barrier, and the waves read their chunks from LDS.
// (Each wave staging its own chunks of x, once faster for 4-bit rows with
// bf16 x, lost once the waves took one row each: q4 layer 20.31 against
// 19.24 us per layer for this kernel at one row per wave.)
// ACC: a stack layer's launch, routing from the accumulators (p.acc)
template <int BITS, int NCH, int NPASS, int XS, bool ACC>
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
  // stacks: the norm's reciprocal, and the logits, from the accumulators
  const float rn = ACC ? acc_rnorm(p.acc, p.E, p.H) : 1.0f;
  if (topk) {
    if constexpr (ACC) {
      if (npl == 2) topk_part_load_acc<2>(p.acc, p.E, wv, rn, lv);
      else topk_part_load_acc<4>(p.acc, p.E, wv, rn, lv);
    } else {
      if (npl == 2) topk_part_load<2>(p.logits, p.E, wv, lv);
      else topk_part_load<4>(p.logits, p.E, wv, lv);
    }
    // the shared gate's weight sigmoid(r * (g . v)), for the combine
    if (ACC && blk == 0 && threadIdx.x == 0)
      p.sigma_out[0] = 1.0f / (1.0f + expf(-(float)acc_entry(p.acc, p.E, p.E) * rn));
    // the other layer parity's accumulators start at zero for the next layer
    if (ACC && p.acc_zero) {
      const int i = blk * kBlock + (int)threadIdx.x;
      if (i < p.acc_zero_n) p.acc_zero[i] = 0.0;
    }
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
    // an entry whose record cannot be read at this width (an id out of
    // range, or the shared expert at another width) reads routed record 0
    // with the routed geometry, so every load stays inside the records, and
    // yields NaN
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
  xpart_store(xp, xw, p.H, rn);  // x = r v in stacks
  __syncthreads();
  if (!active) return;
  if (topk) {
    // each wave needs only its own slot's expert (rank count, no K rounds)
    const int e = wave_uniform(topk_merge_one(tsh, p.E, p.K, slot));
    __builtin_amdgcn_s_setprio(0);
    issue(e);
  }
  __builtin_amdgcn_sched_barrier(0);
  // the first routed workgroup also reports the selection and its weights
  if (topk && blk == 0 && wv == 0) {
    int sel_e = -2;
    uint32_t sel_key = 0, top_key = 0;
    topk_merge(tsh, p.E, p.K, sel_e, sel_key, top_key);
    topk_store(sel_e, topk_merge_weight(tsh, p.K, p.renorm, sel_e, sel_key, top_key), p.K,
               p.idx_out, p.w_out);
  }
  if (fill) gu_store(tile, fill, p.off, m, p.I, row0);
  XStage<BITS, XF32> xs[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = m.li + (j << m.lg);
    xs[j] = xlds_read<BITS, XF32>(xw, c < m.cpr ? c : 0);
  }
  gu_compute(tile, xs, m, p.I, row0, valid, hout);
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
  MOE_LAUNCH(k_topk, dim3(p.T), dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gateup(const GateUpParams &p0, hipStream_t s) {
  GateUpParams p = p0;
  const int nch = nch_for(p.H, p.bits);
  const int rpp = rpp_for(p.H, p.bits);
  // one pass with bf16 x (q4 layer: 4,096 routed waves of one gate and one up
  // row instead of 2,048 of two share the compute after the selection,
  // 20.49 -> 19.24 us per layer); two with fp32 x (16 KiB of x staged per
  // workgroup: the stack 21.2 against 22.7 us with one) and for the
  // host-memory tier (rows read over the link in longer runs)
  const bool one_pass = rpp >= 2 || (p.xsrc == XS_BF16 && !p.rec_src);
  const int npass = clamp_pass(nch, pick_pass(tune().gu, one_pass ? 1 : 2));
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
    const size_t lds = (size_t)(p.H * BITS / 128) * XLds<BITS, XS != XS_BF16>::kWords * 4;      \
    if constexpr (XS == XS_F32) {                                                                \
      if (p.acc) {                                                                               \
        MOE_DISPATCH(nch, npass, MOE_LAUNCH((k_gateup_xl<BITS, NCH_, NP_, XS, true>), grid,      \
                                            dim3(kBlock), lds, s, p));                           \
        break;                                                                                   \
      }                                                                                          \
    }                                                                                            \
    MOE_DISPATCH(nch, npass, MOE_LAUNCH((k_gateup_xl<BITS, NCH_, NP_, XS, false>), grid,       \
                                        dim3(kBlock), lds, s, p));                               \
  } while (0)
  // the accumulators (stacks) come with fp32 x
  if (p.acc && p.xsrc != XS_F32) return hipErrorInvalidValue;
  if (p.bits == 4) {
    if (p.xsrc == XS_BF16) { MOE_GU(4, XS_BF16); } else { MOE_GU(4, XS_F32); }
  } else {
    if (p.xsrc == XS_BF16) { MOE_GU(2, XS_BF16); } else { MOE_GU(2, XS_F32); }
  }
#undef MOE_GU
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

}  // namespace moe_impl
