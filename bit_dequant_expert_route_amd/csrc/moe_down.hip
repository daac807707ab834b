// moe_down.hip -- gfx950 kernels of the down projection: the layer's down/combine
// kernel (with the next stack layer's routing partials), the per-expert down
// kernel and the first stack layer's routing partials.  The dequant scheme and
// memory mapping are those described in moe_kernels.hip.
#include "moe_device.h"
#include "moe_launch.h"

#include <math.h>
#include <stdint.h>

namespace moe_impl {

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
// and the other the rest; their partial sums meet in LDS.  EPI: the launch
// forms the next stack layer's routing inputs (p.nr_acc set).
template <int BITS, int NCH, int NPASS, int MAXK, bool SHARED_IN, bool USE_LDS, int WAVES, bool SPLIT,
          bool EPI>
__global__ __launch_bounds__(64 * WAVES, (MAXK == 1 && BITS == 4) ? 4 : 1) void k_down_combine(DownParams p) {
  constexpr int kThreads = 64 * WAVES;
  static_assert(!SPLIT || WAVES % 2 == 0, "waves pair up");
  // [K (+1)][I]: the SwiGLU outputs, staged once, each code chunk's columns
  // followed by kLdsPad unused floats
  extern __shared__ float hl[];
  constexpr int XSH = USE_LDS ? XS_LDSPAD : XS_F32;
  constexpr int NC = ChunkGeom<BITS>::kCols;
  const int wv = wave_uniform(threadIdx.x >> 6);
  // with the routing partials, block b takes row tile (b mod 8) * (n / 8) +
  // b / 8: blocks are handed to the 8 XCDs in turn, so each XCD gets a
  // contiguous range of tiles (the next layer's router slices of neighbouring
  // tiles share cache lines, which then stay in one XCD's L2; 60-layer q4
  // stack: 21.7 against 22.7 us per layer without it)
  const int nb = (int)gridDim.x;
  const int blk = wave_uniform((EPI && nb % 8 == 0) ? ((int)blockIdx.x % 8) * (nb / 8) + (int)blockIdx.x / 8
                                                    : (int)blockIdx.x);
  const int wave = wave_uniform(SPLIT ? blk * (WAVES / 2) + (wv >> 1) : blk * WAVES + wv);
  const int half = SPLIT ? (wv & 1) : 0;
  const RowMap m = row_map<BITS>(p.I);
  const int row0 = wave * p.rows_per_wave;
  const bool active = row0 < p.H;
  // the next layer's routing inputs (stacks): this workgroup's rows and its
  // slices of the next router and gate (the gate's in the thread that takes
  // its entry), requested first so that they arrive with the rest
  constexpr bool epi = EPI;
  const int wg_rows = (SPLIT ? WAVES / 2 : WAVES) * p.rows_per_wave;
  const int wg_row0 = blk * wg_rows;
  uint4 rpre[4], gpre[4] = {};
  const bool use_pre = epi && slice_fits_pre(p.nr_router_dtype, wg_rows) && (int)threadIdx.x < p.nr_E;
  if (use_pre) {
    if (p.nr_router_tiles)
      slice_prefetch_tiles(p.nr_router_tiles, p.nr_router_dtype, p.nr_E, threadIdx.x, wg_row0, wg_rows, rpre);
    else
      slice_prefetch(p.nr_router, p.nr_router_dtype, p.H, threadIdx.x, wg_row0, wg_rows, rpre);
  }
  const bool gate_pre = epi && slice_fits_pre(p.nr_gate_dtype, wg_rows) && (int)threadIdx.x == p.nr_E % kThreads;
  if (gate_pre) slice_prefetch(p.nr_gate, p.nr_gate_dtype, p.H, 0, wg_row0, wg_rows, gpre);
  // experts in order: the shared one (if here), then the routed ones
  constexpr int SIN = SHARED_IN ? 1 : 0;
  const int n_first = (p.K + SIN + 1) / 2;
  auto mine = [&](int slot) { return !SPLIT || ((slot < n_first) == (half == 0)); };

  // Loads in the order their data are needed (vmcnt counts in order): the
  // selection, the SwiGLU outputs for LDS, the shared expert's rows (known
  // before the selection), then the routed rows once the ids have arrived.
  // Only the LDS fill waits at the barrier, so it no longer waits for the
  // shared rows too (q4 layer 21.01 -> 20.65 us per layer); each expert's
  // rows are consumed as they arrive.  With the routing partials (stacks),
  // whose router slices are already first in the queue, the shared rows go
  // before the SwiGLU outputs (60-layer stack 21.12 -> 21.26 us the other
  // way).
  int ids[MAXK];
  float wk[MAXK];
  if (MAXK == 1 && p.fixed_first) {  // uniform
    ids[0] = 0;
    wk[0] = 1.0f;
  } else {
#pragma unroll
    for (int k = 0; k < MAXK; ++k) {
      ids[k] = k < p.K ? p.idx[k] : -2;
      wk[k] = k < p.K ? p.w[k] : 0.f;
    }
  }
  DnTile<BITS, NCH, NPASS> ts;
  if constexpr (SHARED_IN && EPI) {
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
  if constexpr (SHARED_IN && !EPI) {
    if (mine(0)) down_load(ts, p.shared_rec, p.soff, p.H, m, row0);
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
  // past H are masked where they are loaded and stored; with the routing
  // partials every wave stays for the workgroup's last barrier)
  if (!SPLIT && !active && !epi) return;
  const int hstride = USE_LDS ? lds_stride : p.I;
  const float *hr = USE_LDS ? hl : p.h_routed;
  const float *hs = USE_LDS ? hl + (size_t)p.K * lds_stride : p.h_shared;

  float acc[NPASS];
#pragma unroll
  for (int i = 0; i < NPASS; ++i) acc[i] = 0.f;
  // the shared gate: sigmoid(g . x), from this layer's accumulators in stacks
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
  bool writer = active;
  if constexpr (SPLIT) {
    __shared__ float part[WAVES / 2][NPASS][64];
    if (half) {
#pragma unroll
      for (int i = 0; i < NPASS; ++i) part[wv >> 1][i][lane_id()] = acc[i];
    }
    __syncthreads();
    writer = !half && active;
    if (!writer && !epi) return;
    if (writer) {
#pragma unroll
      for (int i = 0; i < NPASS; ++i) acc[i] += part[wv >> 1][i][lane_id()];
    }
  }
  __shared__ float vrow[64];  // this workgroup's output rows (routing partials)
#pragma unroll
  for (int i = 0; i < NPASS; ++i) {
    const float s = seg_sum(acc[i], m.lg);
    const int r = row0 + i * m.rpp + m.rip;
    if (writer && m.li == 0 && r < p.H) {
      float o = p.h_res[r] + s;
      if constexpr (!SHARED_IN) {
        if (p.y) o = fmaf(sig, p.y[r], o);
      }
      if (EPI && p.nr_upd) o += __uint_as_float((uint32_t)p.nr_upd[r] << 16);  // the next layer's update
      p.out[r] = o;
      if (epi) vrow[r - wg_row0] = o;
    }
  }
  if (epi) {
    __syncthreads();
    routing_partials(p.nr_router, p.nr_router_dtype, p.nr_gate, p.nr_gate_dtype, p.nr_E, p.H, vrow,
                     wg_row0, wg_rows, p.nr_acc, (int)blockIdx.x % kAccCopies, kThreads, rpre, use_pre,
                     gpre, gate_pre);
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
  // unreadable entries (as in k_gateup_xl) read routed record 0 and yield NaN
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
// the first stack layer's routing accumulators: v = h + u for this
// workgroup's kPartialsRows rows, then its routing partials
// ---------------------------------------------------------------------------
constexpr int kPartialsRows = 16;

__global__ __launch_bounds__(kBlock) void k_partials(PartialsParams p) {
  __shared__ float vrow[kPartialsRows];
  const int r0 = blockIdx.x * kPartialsRows;
  uint4 rpre[4];
  const bool use_pre = slice_fits_pre(p.router_dtype, kPartialsRows) && (int)threadIdx.x < p.E;
  if (use_pre) {
    if (p.router_tiles)
      slice_prefetch_tiles(p.router_tiles, p.router_dtype, p.E, threadIdx.x, r0, kPartialsRows, rpre);
    else
      slice_prefetch(p.router, p.router_dtype, p.H, threadIdx.x, r0, kPartialsRows, rpre);
  }
  uint4 gpre[4] = {};
  const bool gate_pre = slice_fits_pre(p.gate_dtype, kPartialsRows) && (int)threadIdx.x == p.E % kBlock;
  if (gate_pre) slice_prefetch(p.gate, p.gate_dtype, p.H, 0, r0, kPartialsRows, gpre);
  if (threadIdx.x < kPartialsRows) {
    const int r = r0 + threadIdx.x;
    float v = p.h[r];
    if (p.upd) v += __uint_as_float((uint32_t)p.upd[r] << 16);
    p.v_out[r] = v;
    vrow[threadIdx.x] = v;
  }
  __syncthreads();
  routing_partials(p.router, p.router_dtype, p.gate, p.gate_dtype, p.E, p.H, vrow, r0,
                   kPartialsRows, p.acc, (int)blockIdx.x % kAccCopies, kBlock, rpre, use_pre, gpre,
                   gate_pre);
}

hipError_t launch_partials(const PartialsParams &p, hipStream_t s) {
  if (p.H % kPartialsRows) return hipErrorInvalidValue;
  MOE_LAUNCH(k_partials, dim3(p.H / kPartialsRows), dim3(kBlock), 0, s, p);
  return hipGetLastError();
}


// the combine kernel's shape: rows per wave, whether the SwiGLU outputs go
// through LDS, and the workgroup form (eight waves, or split pairs)
struct CombineShape {
  int rows_per_wave;
  bool use_lds, eight, split;
  size_t lds;
  int wg_rows() const { return (eight ? 8 : (split ? 2 : 4)) * rows_per_wave; }
};

static CombineShape combine_shape(int H, int I, int bits, int n_vectors) {
  CombineShape c;
  const int nch = nch_for(I, bits);
  const int rpp = rpp_for(I, bits);
  const int npass = clamp_pass(nch, pick_pass(tune().dn, rpp >= 2 ? 1 : 2));
  c.rows_per_wave = npass * rpp;
  const int waves = (H + c.rows_per_wave - 1) / c.rows_per_wave;
  // the SwiGLU outputs go through LDS (padded per code chunk) when they fit
  // in 64 KiB
  const int nc = 128 / bits;
  const size_t hbytes = (size_t)n_vectors * (I / nc) * (nc + kLdsPad) * sizeof(float);
  c.use_lds = hbytes <= 65536;
  c.lds = c.use_lds ? hbytes : 0;
  // eight-wave workgroups when there are enough waves for one per CU (q4
  // layer: 20.85 against 21.15 us; with 1024 waves, half the CUs would idle)
  c.eight = c.use_lds && waves >= 8 * kCUs;
  // otherwise (fewer rows) two waves share each set of rows, splitting the
  // experts, so that the grid still has waves to hide latency with
  c.split = c.use_lds && !c.eight;
  return c;
}

bool combine_takes_partials(int H, int I, int bits, int n_vectors) {
  const CombineShape c = combine_shape(H, I, bits, n_vectors);
  const int r = c.wg_rows();
  return c.use_lds && r <= 64 && r % 8 == 0 && H % r == 0;
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
    const CombineShape cs = combine_shape(p.H, p.I, bits, p.K + (shared_in ? 1 : 0));
    const int waves = (p.H + p.rows_per_wave - 1) / p.rows_per_wave;
    const bool k4 = p.K <= 4;
    const bool eight = cs.eight, split = cs.split;
    const size_t lds = cs.lds;
    const dim3 grid(eight ? (waves + 7) / 8 : (split ? (waves + 1) / 2 : (waves + 3) / 4));
    // the routing partials need whole workgroup row tiles of 8..64 rows and
    // the SwiGLU outputs in LDS
    if (p.nr_acc && (!shared_in || !combine_takes_partials(p.H, p.I, bits, p.K + 1)))
      return hipErrorInvalidValue;
    const bool epi = p.nr_acc != nullptr;
    // (the partials epilogue is built for stack layers: shared expert in)
#define MOE_DC(BITS, MAXK, SIN)                                                                       \
  do {                                                                                                \
    if constexpr (SIN) {                                                                              \
      if (eight && epi) {                                                                             \
        MOE_DISPATCH(nch, npass, MOE_LAUNCH((k_down_combine<BITS, NCH_, NP_, MAXK, SIN, true, 8, false, true>), \
                                            grid, dim3(512), lds, s, p));                             \
        break;                                                                                        \
      }                                                                                               \
      if (split && epi) {                                                                             \
        MOE_DISPATCH(nch, npass, MOE_LAUNCH((k_down_combine<BITS, NCH_, NP_, MAXK, SIN, true, 4, true, true>), \
                                            grid, dim3(kBlock), lds, s, p));                          \
        break;                                                                                        \
      }                                                                                               \
    }                                                                                                 \
    if (eight)                                                                                        \
      MOE_DISPATCH(nch, npass, MOE_LAUNCH((k_down_combine<BITS, NCH_, NP_, MAXK, SIN, true, 8, false, false>), \
                                          grid, dim3(512), lds, s, p));                               \
    else if (split)                                                                                   \
      MOE_DISPATCH(nch, npass, MOE_LAUNCH((k_down_combine<BITS, NCH_, NP_, MAXK, SIN, true, 4, true, false>), \
                                          grid, dim3(kBlock), lds, s, p));                            \
    else                                                                                              \
      MOE_DISPATCH(nch, npass, MOE_LAUNCH((k_down_combine<BITS, NCH_, NP_, MAXK, SIN, false, 4, false, false>), \
                                          grid, dim3(kBlock), 0, s, p));                              \
  } while (0)
    // one expert and no shared one (the linear-attention block's output
    // projection): tiles for one expert only, so the kernel keeps few
    // registers and its waves fit the CUs in one round
    const bool k1 = p.K == 1 && !shared_in;
    if (p.fixed_first && !k1) return hipErrorInvalidValue;
    if (bits == 4) {
      if (shared_in) { if (k4) MOE_DC(4, 4, true); else MOE_DC(4, 8, true); }
      else { if (k1) MOE_DC(4, 1, false); else if (k4) MOE_DC(4, 4, false); else MOE_DC(4, 8, false); }
    } else {
      if (shared_in) { if (k4) MOE_DC(2, 4, true); else MOE_DC(2, 8, true); }
      else { if (k1) MOE_DC(2, 1, false); else if (k4) MOE_DC(2, 4, false); else MOE_DC(2, 8, false); }
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

}  // namespace moe_impl
