// moe_internal.h -- parameter blocks and launchers shared by the C ABI layer
// (moe_api.cpp) and the gfx950 kernels (moe_kernels.hip).  Library-internal.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe_impl {

constexpr int kGroup = 64;
constexpr int kMaxK = 8;
constexpr int kMaxE = 1024;
constexpr int kMaxDim = 8192;
constexpr int kMaxTokens = 64;
constexpr int kSharedId = -1;          // MOE_SHARED
constexpr int kBlock = 256;            // threads per workgroup (4 waves)
constexpr int kCUs = 256;              // compute units of an MI355X

// where a kernel reads its activation vector from
enum XSrc : int {
  XS_BF16 = 0,   // bf16 [H] in global memory
  XS_F32 = 1,    // fp32 [H] in global memory
  XS_NORM = 2,   // x = rmsnorm(h + u), computed per workgroup into LDS
  XS_LDSPAD = 3, // fp32 in LDS, each code chunk's columns followed by kLdsPad
                 // floats, the first holding the chunk's column sum (the pad
                 // spreads the lanes' 16-byte reads over banks)
};
constexpr int kLdsPad = 4;

// byte offsets of a record's sections
struct RecOffsets {
  size_t gate_codes, up_codes, down_codes, gate_sb, up_sb, down_sb, total;
};
RecOffsets record_offsets(int hidden, int inter, int bits);

// ---------------------------------------------------------------------------
// K1: router rows + shared-gate dot + (optionally) the shared expert's
//     gate/up/SwiGLU rows.  One launch per layer.
// ---------------------------------------------------------------------------
struct HeadParams {
  int H, I, E, T;                 // T tokens (router + gate only when T > 1)
  int router_dtype;               // 0 f32, 1 bf16
  const void *router;             // [E][H]
  int gate_dtype;
  const void *gvec;               // [H]
  int xsrc;                       // XSrc
  const void *x;                  // [T][H] (XS_BF16 / XS_F32)
  const float *h_in;              // XS_NORM: [H] residual before the update
  const uint16_t *upd;            // XS_NORM: [H] bf16 update, may be null
  float *logits;                  // [T][E]
  float *sigma;                   // [T]
  float *x_out;                   // XS_NORM: fp32 x written by workgroup 0
  float *hres_out;                // XS_NORM: fp32 h + u written by workgroup 0
  // shared expert (only when n_shared_waves > 0)
  const uint8_t *shared_rec;
  int bits_shared;
  RecOffsets soff;
  float *h_shared;                // [I]
  int n_router_blocks;
  int n_shared_waves;
  int shared_rows_per_wave;
  // bf16 x staged once for the routed experts' gate/up (written by one wave
  // when non-null): pairs [chunks][pairs per chunk] u32, sums [chunks][2]
  int bits_routed;
  uint32_t *xs_pairs;
  float *xs_sums;
  int xs_pair_stride, xs_sum_stride;  // per token (u32 / floats); one stager unit per token
};
hipError_t launch_head(const HeadParams &p, hipStream_t s);

// ---------------------------------------------------------------------------
// token batches: top-K of every token, then the (token, expert) pairs sorted
// by expert (token order kept inside an expert) into groups
// ---------------------------------------------------------------------------
struct RouteGroupParams {
  const float *logits;            // [T][E]
  int T, E, K, renorm;
  int selected;                   // 1: idx holds the selection; only group
  int32_t *idx;                   // [T][K]
  float *w;                       // [T][K]
  int32_t *g_count;               // [1]  number of distinct experts U
  int32_t *g_expert;              // [U]  ascending expert id
  int32_t *g_start;               // [U + 1] first position of each group in g_pair
  int32_t *g_pair;                // [T K] pair index t K + k, grouped
};
hipError_t launch_route_group(const RouteGroupParams &p, hipStream_t s);

// gate/up and down over the groups: each wave keeps one expert's weight rows
// in registers and applies them to every token of the group; the shared
// expert is one more group holding every token
struct GroupedParams {
  int H, I, E, K, T;
  int bits;                       // width of the experts this launch covers
  const uint8_t *experts;
  size_t stride;
  const uint8_t *shared_rec;
  RecOffsets off, soff;
  const int32_t *g_count, *g_expert, *g_start, *g_pair;
  int do_routed, do_shared;
  // gate/up input
  int xsrc;                       // XS_BF16 or XS_F32
  const void *x;                  // [T][H]
  const uint32_t *xs_pairs;       // staged bf16 x per token, or null
  const float *xs_sums;
  int xs_pair_stride, xs_sum_stride;
  // SwiGLU outputs (gate/up writes them, down reads them)
  float *h_routed;                // [T K][I] by pair
  float *h_shared;                // [T][I]
  // down outputs
  float *y_routed;                // [T K][H] by pair
  float *y_shared;                // [T][H]
  int rows_per_wave, tiles;       // set by the launcher (tiles of four waves)
  int tok_batch;                  // tokens staged in LDS at a time (launcher)
  int shared_split;               // token ranges of the shared expert's items (launcher)
  // gate/up only: the selection [T][K]; when set (T K <= kGroupInKernel) the
  // kernel groups the pairs itself and its workgroup 0 writes g_* for the
  // down kernel, instead of a grouping launch before it
  const int32_t *group_idx;
};
constexpr int kGroupInKernel = 128;
hipError_t launch_gateup_grouped(const GroupedParams &p, hipStream_t s);
hipError_t launch_down_grouped(const GroupedParams &p, hipStream_t s);

// out[t] = h_res[t] + sum_k w[t][k] y_routed[t K + k] + sigma[t] y_shared[t]
struct CombineTokensParams {
  int H, K, T;
  const float *h_res, *y_routed, *w, *y_shared, *sigma;
  float *out;
};
hipError_t launch_combine_tokens(const CombineTokensParams &p, hipStream_t s);

// ---------------------------------------------------------------------------
// top-K + softmax weights from logits (stand-alone routing entry point)
// ---------------------------------------------------------------------------
struct TopkParams {
  const float *logits;  // [T][E]
  int T, E, K, renorm;
  int32_t *idx;         // [T][K]
  float *w;             // [T][K]
};
hipError_t launch_topk(const TopkParams &p, hipStream_t s);

// ---------------------------------------------------------------------------
// K2: gate/up + SwiGLU for a list of experts (explicit ids, or the top-K of
//     device logits computed by every wave)
// ---------------------------------------------------------------------------
struct GateUpParams {
  int H, I, E, K, renorm;
  int bits;                       // width of the listed experts
  const uint8_t *experts;
  size_t stride;
  const uint8_t *shared_rec;
  int shared_ok;                  // shared record has this width
  RecOffsets off;                 // routed record offsets (bits)
  RecOffsets soff;                // shared record offsets (bits_shared)
  const int32_t *ids;             // [n] explicit ids, or null -> top-K of logits
  int n;                          // list length (== K in top-K mode)
  const float *logits;            // [E] (top-K mode)
  int32_t *idx_out;               // top-K mode: written by wave 0 (may be null)
  float *w_out;
  int xsrc;                       // XS_BF16 or XS_F32
  const void *x;                  // [H]
  float *h_out;                   // [n][I]
  // the shared expert's gate/up in the same launch (same width): its
  // workgroups come after the routed ones and need no routing
  int with_shared;
  float *h_shared_out;            // [I]
  int n_shared_blocks;            // set by the launcher
  int rows_per_wave;
  int waves_per_expert;
  // expert tier: per list entry, the address of the record to read (a cache
  // slot, or the record in host memory on a miss) and where to write the
  // rows read (the slot on a miss, else 0); null outside the tier path
  const uint64_t *rec_src;        // [n]
  const uint64_t *rec_fill;       // [n]
  // with rec_fill: workgroups after all others copy the down section of every
  // entry that has a fill target (set by the launcher)
  int n_copy_blocks, copy_blocks_per_entry;
  // stacks: the routing comes from accumulators ([kAccCopies][acc_stride(E)],
  // see kAccCopies) instead of logits, x is v scaled by the norm's reciprocal
  // (p.x holds v, fp32), the routed workgroups zero acc_zero (the other
  // layer parity's accumulators, acc_zero_n doubles), and the first writes
  // the shared gate's sigmoid to sigma_out
  const double *acc;
  double *acc_zero;
  int acc_zero_n;
  float *sigma_out;
};
hipError_t launch_gateup(const GateUpParams &p, hipStream_t s);

// ---------------------------------------------------------------------------
// K3: down projection.  COMBINE: every wave takes all K routed experts (ids
//     and weights from device memory) plus the shared expert (weight sigma)
//     for its output rows and writes out = h_res + sum.  Y: one expert per
//     wave, y[slot][o] written.
// ---------------------------------------------------------------------------
struct DownParams {
  int H, I, E;
  int bits_r, bits_s;
  const uint8_t *experts;
  size_t stride;
  const uint8_t *shared_rec;
  RecOffsets off, soff;
  int combine;                    // 1 COMBINE, 0 Y
  // COMBINE
  const int32_t *idx;             // [K]
  const float *w;                 // [K]
  int K;
  // K == 1 with weight 1 on expert 0, known to the launcher (the
  // linear-attention block's output projection): idx and w are not read, so
  // the rows are requested without waiting for an id
  int fixed_first;
  const float *sigma;             // [1]
  const float *h_routed;          // [K][I]
  const float *h_shared;          // [I]
  const float *h_res;             // [H]
  float *out;                     // [H]
  // Y
  const int32_t *ids;             // [n]
  int n;
  const float *h;                 // [n][I]
  float *y;                       // [n][H]
  int shared_ok;
  int rows_per_wave;
  int waves_per_expert;           // Y mode
  // stacks (COMBINE mode): the next layer's routing inputs formed here from
  // this launch's output rows.  With nr_acc set, the output is
  // v = out + u_next (u_next may be null) and every workgroup adds, for its
  // rows, the partial dots of v with each router row and the gate vector and
  // the partial sum of v^2 into copy (block mod kAccCopies) of nr_acc.
  const void *nr_router;          // [nr_E][H]
  const void *nr_router_tiles;    // the same in column tiles (moe_router_tile) or null
  int nr_router_dtype;
  const void *nr_gate;            // [H]
  int nr_gate_dtype;
  const uint16_t *nr_upd;         // [H] bf16 or null
  double *nr_acc;                 // [kAccCopies][acc_stride(nr_E)] or null
  int nr_E;
};
hipError_t launch_down(const DownParams &p, hipStream_t s);
// whether a combine launch of this shape (n_vectors = K routed + shared) can
// form the next layer's routing partials (its workgroups stage the SwiGLU
// outputs in LDS and cover 8..64 rows)
bool combine_takes_partials(int H, int I, int bits, int n_vectors);

// Routing accumulators of a stack layer: entry e < E the router dot of row e
// with v, entry E the gate dot, entry E + 1 the sum of v^2; each summed in fp64
// over kAccCopies copies that the producing workgroups spread their atomic
// additions over.  The router logits are r * dot and the gate sigmoid's
// argument r * gate, with r = 1 / sqrt(sum / H + 1e-6).  Copy c is a run of
// acc_stride(E) doubles (E + 2 rounded up to whole 128-byte lines), so that the
// lanes of a wave, taking consecutive entries, add into and read consecutive
// addresses.  Every gate/up workgroup reads all copies, while additions to
// one address wait on each other: four copies (60-layer q4 stack, per layer:
// 16 copies 23.1 us, 8 copies 22.0, 4 copies 21.8).
constexpr int kAccCopies = 4;
__host__ __device__ constexpr int acc_stride(int E) { return (E + 2 + 15) / 16 * 16; }
inline size_t acc_doubles(int E) { return (size_t)acc_stride(E) * kAccCopies; }

// the first layer's routing accumulators: v = h + u (written to v_out) and
// the partial dots of v, from every workgroup's rows
struct PartialsParams {
  int H, E;
  const float *h;
  const uint16_t *upd;            // [H] bf16 or null
  float *v_out;
  const void *router;
  const void *router_tiles;       // column tiles (moe_router_tile) or null
  int router_dtype;
  const void *gate;
  int gate_dtype;
  double *acc;
};
hipError_t launch_partials(const PartialsParams &p, hipStream_t s);

// out[t][e][0..8) = router[e][8t..8t+8) (element size esz)
hipError_t launch_router_tile(const void *router, int E, int H, int esz, void *out, hipStream_t s);

// ---------------------------------------------------------------------------
// expert tier: top-K of one token's logits, then each selected expert's cache
// slot from the device-resident state (least recently used slot not taken by
// this token on a miss), and the record address every expert kernel reads
// ---------------------------------------------------------------------------
struct TierState {                // device layout of the tier state
  uint32_t tick, pad[1];
  unsigned long long hits, misses, bytes;
  // followed at kTierOwnerOff by owner[n_slots] int32 (expert in the slot or
  // -1), then last_use[n_slots] uint32 (tick of its last use, 0 = never)
};
constexpr size_t kTierOwnerOff = 64;
struct TierRouteParams {
  const float *logits;            // [E]
  int E, K, renorm, n_slots;
  uint8_t *state;
  const uint8_t *host_dev;        // device address of the host records
  uint8_t *cache;
  size_t stride, record_bytes;
  int32_t *idx;                   // [K] expert ids
  float *w;                       // [K]
  int32_t *slot;                  // [K] slot, or -1 for an invalid selection
  uint64_t *rec_src;              // [K]
  uint64_t *rec_fill;             // [K]
};
hipError_t launch_tier_route(const TierRouteParams &p, hipStream_t s);
hipError_t launch_tier_reset(uint8_t *state, int n_slots, hipStream_t s);

struct CombineParams {
  int H, K;
  const float *h_res, *y, *w, *y_shared, *sigma;
  float *out;
};
hipError_t launch_combine(const CombineParams &p, hipStream_t s);

struct FillParams {
  uint8_t *dst;
  size_t stride;
  int n;
  uint64_t seed;
  int layer, first_expert, H, I, bits;
  double scale_lo, scale_hi, bias_lo, bias_hi;
  RecOffsets off;
};
hipError_t launch_fill(const FillParams &p, hipStream_t s);

hipError_t launch_zero(void *ptr, size_t bytes, hipStream_t s);

// Kernel timing: while `start` is set, each launcher's kernel dispatch records
// these two events itself (the dispatch packet's own begin and end), so the
// elapsed time is the kernel's execution time with no marker packets around it.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
extern thread_local LaunchEvents g_launch_events;

#define MOE_LAUNCH(kern, grid, block, lds, stream, ...)                                      \
  do {                                                                                       \
    if (::moe_impl::g_launch_events.start)                                                   \
      hipExtLaunchKernelGGL(kern, grid, block, lds, stream, ::moe_impl::g_launch_events.start, \
                            ::moe_impl::g_launch_events.stop, 0, __VA_ARGS__);               \
    else                                                                                     \
      hipLaunchKernelGGL(kern, grid, block, lds, stream, __VA_ARGS__);                       \
  } while (0)

// gated delta-rule decode step (moe_gdn.hip)
struct GdnParams {
  int n_sh;                       // sequences * heads
  int d_k, d_v;                   // d_k in {16, 32, 64, 128, 256}
  const float *q, *k;             // [n_sh][d_k]
  const float *v;                 // [n_sh][d_v]
  const float *alpha, *beta;      // [n_sh]
  float *state;                   // [n_sh][d_v][d_k], updated in place
  float *out;                     // [n_sh][d_v]
  // 1: q and k are raw projections, scaled here to unit length per head
  // (eps 1e-6 under the root), and alpha, beta are logits, made sigmoids here
  int prep;
};
hipError_t launch_gdn_step(const GdnParams &p, hipStream_t s);

// the projections of a linear-attention block: x = RMSNorm(h) formed per
// workgroup in LDS, then the rows of W_q, W_k (gate, up of rec_qko), W_v and
// the 2 n_heads gate rows (gate, first rows of up of rec_vab) -> proj
struct GdnInParams {
  int H, D, n_heads, bits;
  const float *h;                 // [H]
  const uint8_t *rec_qko, *rec_vab;
  RecOffsets off;                 // record offsets at (H, D, bits)
  float *proj;                    // [3 D + 2 n_heads]: q, k, v, alpha and beta logits
  // one routed entry of weight 1 and a zero shared gate, for the output
  // projection's down/combine launch (written by workgroup 0)
  int32_t *one_idx;
  float *one_w, *zero_sigma;
  int rows_per_wave;              // set by the launcher
};
hipError_t launch_gdn_in(const GdnInParams &p, hipStream_t s);

// workspace of moe_layer_decode_noalloc: a device array of this many bytes
// per GPU (moe_util.hip); *out receives the current device's address of it
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
hipError_t noalloc_scratch(void **out);

// bytes of the staged-x buffers for a row of `cols` columns at `bits`
size_t xstage_pair_bytes(int cols, int bits);
size_t xstage_sum_bytes(int cols, int bits);
hipError_t launch_copy_f32(float *dst, const float *src, int n, hipStream_t s);

}  // namespace moe_impl
