// moe_batch.hip -- gfx950 kernels of the batched (grouped) path: routing of a
// token batch into per-expert groups, grouped gate/up and down, and the
// per-token combine.
#include "moe_device.h"
#include "moe_launch.h"

#include <math.h>
#include <stdint.h>

#include <type_traits>

namespace moe_impl {

// ---------------------------------------------------------------------------
// token batches
// ---------------------------------------------------------------------------
// One workgroup: the top-K of every token (wave w takes tokens w, w + 4, ...),
// then a counting sort of the T*K (token, expert) pairs by expert id with the
// pair order kept inside an expert.  P = T*K <= 512 and the ranks are plain
// counts over the pairs, so the result does not depend on thread timing.
constexpr int kGroupBlock = 1024;  // one wave per token for up to 16 tokens at a time

// Counting sort of the P (token, expert) pairs whose experts are in pe[] (LDS,
// P entries, visible to the whole workgroup) by expert id, pair order kept
// inside an expert: g_pair holds the pairs grouped, g_expert the U distinct
// experts ascending, g_start[g] the first position of group g (g_start[U] =
// P), g_count[0] = U.  pless, pfirst and n_first are LDS scratch (n_first
// zeroed before the caller's barrier).  The ranks are plain counts over the
// pairs, so the result does not depend on thread timing.  The outputs may be
// in LDS or in global memory; the caller synchronises before reading them.
__device__ __forceinline__ void group_pairs(const int *pe, int P, int *pless, unsigned char *pfirst,
                                            int &n_first, int32_t *g_pair, int32_t *g_expert,
                                            int32_t *g_start, int32_t *g_count) {
  const int nt = (int)blockDim.x;
  int mine = 0;
  for (int q = threadIdx.x; q < P; q += nt) {
    const int e = pe[q];
    int less = 0, before = 0;
    for (int r = 0; r < P; ++r) {
      const int f = pe[r];
      less += f < e;
      before += (r < q) & (f == e);
    }
    g_pair[less + before] = q;
    pless[q] = less;
    pfirst[q] = before == 0;
    mine += before == 0;
  }
  atomicAdd(&n_first, mine);
  __syncthreads();
  for (int q = threadIdx.x; q < P; q += nt) {
    if (!pfirst[q]) continue;
    const int e = pe[q];
    int g = 0;
    for (int r = 0; r < P; ++r) g += pfirst[r] & (pe[r] < e);
    g_expert[g] = e;
    g_start[g] = pless[q];
  }
  if (threadIdx.x == 0) {
    g_count[0] = n_first;
    g_start[n_first] = P;
  }
}

// One workgroup: the top-K of every token (wave w takes tokens w, w + 4, ...)
// unless the selection is given, then the grouping of the T*K pairs.
__global__ __launch_bounds__(kGroupBlock) void k_route_group(RouteGroupParams p) {
  __shared__ int pe[kMaxTokens * kMaxK];
  __shared__ int pless[kMaxTokens * kMaxK];
  __shared__ unsigned char pfirst[kMaxTokens * kMaxK];
  __shared__ int n_first;
  const int wv = threadIdx.x >> 6, lane = lane_id();
  if (threadIdx.x == 0) n_first = 0;
  if (p.selected) {  // the selection is in p.idx already (k_topk)
    for (int q = threadIdx.x; q < p.T * p.K; q += kGroupBlock) pe[q] = p.idx[q];
  } else {
    for (int t = wv; t < p.T; t += kGroupBlock / 64) {
      float v[kTopkNpl];
      topk_load(p.logits + (size_t)t * p.E, p.E, v);
      int e;
      float w;
      topk_select(v, p.E, p.K, p.renorm, e, w);
      topk_store(e, w, p.K, p.idx + (size_t)t * p.K, p.w + (size_t)t * p.K);
      if (lane < p.K) pe[t * p.K + lane] = e;
    }
  }
  __syncthreads();
  group_pairs(pe, p.T * p.K, pless, pfirst, n_first, p.g_pair, p.g_expert, p.g_start, p.g_count);
}


// The grouped gate/up kernel's own grouping (batches of at most
// kGroupInKernel pairs): every workgroup sorts the pairs into LDS from the
// selection, so no grouping launch sits between the top-K and the gate/up.
// (a multiple of 16 bytes: the kernel's dynamic LDS, read with 16-byte
// loads, starts right after it)
struct alignas(16) GroupLds {
  int pe[kGroupInKernel], pless[kGroupInKernel];
  int32_t pair[kGroupInKernel], expert[kGroupInKernel], start[kGroupInKernel + 1], count;
  unsigned char pfirst[kGroupInKernel];
  int n_first;
};
static_assert(sizeof(GroupLds) % 16 == 0, "keeps the dynamic LDS after it 16-byte aligned");

// The groups as the grouped kernels read them: in global memory (written by
// k_route_group or by the gate/up kernel's workgroup 0), or in the gate/up
// kernel's LDS.  Two types rather than one pointer that may point to either,
// so that the LDS reads compile to LDS instructions: a flat load would also
// count against the vector memory counter and wait for the weight rows
// requested ahead of it.
struct GlobalGroups {
  const GroupedParams &p;
  __device__ int expert(int g) const { return p.g_expert[g]; }
  __device__ int start(int g) const { return p.g_start[g]; }
  __device__ int pair(int i) const { return p.g_pair[i]; }
};
struct LdsGroups {
  const GroupLds &gl;
  __device__ int expert(int g) const { return gl.expert[g]; }
  __device__ int start(int g) const { return gl.start[g]; }
  __device__ int pair(int i) const { return gl.pair[i]; }
};

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

template <class Groups>
__device__ __forceinline__ GroupRef item_ref(const GroupedParams &p, const Groups &gv, int item,
                                             int U, int &tile) {
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
    r.id = wave_uniform(gv.expert(g));
    const int s0 = wave_uniform(gv.start(g));
    r.n = wave_uniform(gv.start(g + 1)) - s0;
    r.pair = lane < r.n ? gv.pair(s0 + lane) : 0;
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
// GL: the kernel groups the (token, expert) pairs itself, into LDS
// (p.group_idx set, at most kGroupInKernel pairs)
template <int BITS, int NCH, int NPASS, int XS, bool GL>
__global__ __launch_bounds__(kBlock) void k_gateup_grouped(GroupedParams p) {
  extern __shared__ uint32_t lds_x[];
  constexpr bool XF32 = XS != XS_BF16;
  using Stage = XStage<BITS, XF32>;
  constexpr int CS = lds_chunk_words<Stage>();
  const int wv = wave_uniform(threadIdx.x >> 6);
  __shared__ GroupLds gl;
  int U = 0;
  if (GL && p.do_routed) {  // launch-uniform
    const int P = p.T * p.K;
    if (threadIdx.x == 0) gl.n_first = 0;
    for (int q = threadIdx.x; q < P; q += kBlock) gl.pe[q] = p.group_idx[q];
    __syncthreads();
    group_pairs(gl.pe, P, gl.pless, gl.pfirst, gl.n_first, gl.pair, gl.expert, gl.start, &gl.count);
    __syncthreads();
    U = gl.count;
    if (blockIdx.x == 0) {  // the groups for the down kernel (the workspace
                            // arrays a grouping launch would have written)
      int32_t *g_pair = const_cast<int32_t *>(p.g_pair), *g_expert = const_cast<int32_t *>(p.g_expert);
      int32_t *g_start = const_cast<int32_t *>(p.g_start), *g_count = const_cast<int32_t *>(p.g_count);
      for (int q = threadIdx.x; q < P; q += kBlock) {
        g_pair[q] = gl.pair[q];
        if (q < U) g_expert[q] = gl.expert[q];
      }
      for (int q = threadIdx.x; q <= U; q += kBlock) g_start[q] = gl.start[q];
      if (threadIdx.x == 0) g_count[0] = U;
    }
  } else if (p.do_routed) {
    U = wave_uniform(p.g_count[0]);
  }
  using Groups = typename std::conditional<GL, LdsGroups, GlobalGroups>::type;
  const Groups gv = [&] {
    if constexpr (GL) return LdsGroups{gl};
    else return GlobalGroups{p};
  }();
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
    r = item_ref(p, gv, item < n_items ? item : 0, U, tile);
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
  const GlobalGroups gv{p};
  const int n_items = n_work_items(p, U);
  const RowMap m = row_map<BITS>(p.I);
  const int tok_floats = (p.I / NC) * PC;
  DnTile<BITS, NCH, NPASS> next;
  GroupRef ngr;
  int nrow0 = 0;
  auto fetch = [&](int item, DnTile<BITS, NCH, NPASS> &t, GroupRef &r, int &row0) {
    int tile;
    r = item_ref(p, gv, item < n_items ? item : 0, U, tile);
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
    if (p.group_idx)                                                                           \
      MOE_DISPATCH_G(nch, npass, MOE_LAUNCH((k_gateup_grouped<BITS, NCH_, NP_, XS, true>), grid, \
                                            dim3(kBlock), lds, s, p));                         \
    else                                                                                       \
      MOE_DISPATCH_G(nch, npass, MOE_LAUNCH((k_gateup_grouped<BITS, NCH_, NP_, XS, false>), grid, \
                                            dim3(kBlock), lds, s, p));                         \
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
