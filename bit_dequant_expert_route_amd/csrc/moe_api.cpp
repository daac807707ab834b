// moe_api.cpp -- the C ABI of libmoe: argument checks, workspace layout and
// the sequencing of the gfx950 kernels.  Every check runs before anything is
// enqueued; no call allocates, copies or synchronises.
//
// The layer runs as three launches with no host round trip in between
// (openclawradar.com (ja), "Flash-MoE: running the 397B parameter Qwen model
// on a MacBook Pro in pure C/Metal", section "Deferred GPU expert compute":
// the expert pass is queued without waiting):
//   K1 router rows + shared-gate dot + shared expert gate/up/SwiGLU
//   K2 top-K of the logits (every wave) + routed gate/up/SwiGLU
//   K3 routed (and shared) down projections + combine + residual
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../../include/moe.h"
#include "moe_internal.h"

using namespace moe_impl;

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

int hip_fail(hipError_t e, const char *what) {
  return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// kernel timing state of this thread (moe_profile_begin / moe_profile_end)
struct Prof {
  bool on = false;
  int cap = 0, n = 0;
  std::vector<hipEvent_t> ev;  // two per launch
  std::vector<int> ids;
};
thread_local Prof g_prof;

bool prof_active(hipStream_t s) {
  if (!g_prof.on || g_prof.n >= g_prof.cap) return false;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return false;
  return true;
}

// MOE_DEBUG=1: every launch outside stream capture is followed by a stream
// synchronisation, so that a fault or launch error is reported by the call
// (and the launch) that caused it
bool debug_sync() {
  static const bool on = [] {
    const char *e = getenv("MOE_DEBUG");
    return e && e[0] == '1';
  }();
  return on;
}

hipError_t debug_check(hipStream_t s, hipError_t e) {
  if (e != hipSuccess || !debug_sync()) return e;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return e;
  const hipError_t se = hipStreamSynchronize(s);
  return se != hipSuccess ? se : hipGetLastError();
}

// launch `fn` (one kernel) so that its dispatch records a pair of events
template <class F>
hipError_t timed(hipStream_t s, int id, F &&fn) {
  if (!prof_active(s)) return debug_check(s, fn());
  const int i = g_prof.n;
  g_launch_events.start = g_prof.ev[2 * i];
  g_launch_events.stop = g_prof.ev[2 * i + 1];
  const hipError_t e = fn();
  g_launch_events = LaunchEvents{};
  if (e != hipSuccess) return e;
  g_prof.ids[i] = id;
  g_prof.n = i + 1;
  return debug_check(s, hipSuccess);
}

size_t up256(size_t n) { return (n + 255u) / 256u * 256u; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool dim_ok(int d) { return d >= 64 && d <= kMaxDim && d % kGroup == 0; }

// ---------------------------------------------------------------------------
// workspace layout for one layer call
// ---------------------------------------------------------------------------
struct WsLayout {
  size_t logits, sigma, h_routed, h_shared, y_shared, x_stage, hres_stage, xs_pairs, xs_sums,
      h_pong, acc, y_routed, g_count, g_expert, g_start, g_pair, ids, rec_src, gdn_proj,
      gdn_o, gdn_h, gdn_const, total;
  size_t xs_pair_stride, xs_sum_stride;  // per token, in u32 / floats
};

// gdn_D / gdn_heads: the widest linear-attention block of a stack (0: none)
WsLayout ws_layout(const moe_layer_t *L, int T, int n_layers, int gdn_D = 0, int gdn_heads = 0) {
  WsLayout w;
  size_t o = 0;
  const size_t E = L->n_experts, K = L->top_k, I = L->inter, H = L->hidden;
  const size_t rows_h = (size_t)T * K > (size_t)kMaxTokens ? (size_t)T * K : (size_t)kMaxTokens;
  w.logits = o; o += up256(4 * (size_t)T * E);
  w.sigma = o; o += up256(4 * (size_t)T);
  w.h_routed = o; o += up256(4 * rows_h * I);
  w.h_shared = o; o += up256(4 * (size_t)T * I);
  w.y_shared = o; o += up256(4 * (size_t)T * H);
  w.x_stage = o; o += up256(4 * H);
  w.hres_stage = o; o += up256(4 * H);
  // staged bf16 x, one block per token
  w.xs_pair_stride = up256(xstage_pair_bytes(L->hidden, L->bits_routed)) / 4;
  w.xs_sum_stride = up256(xstage_sum_bytes(L->hidden, L->bits_routed)) / 4;
  w.xs_pairs = o; o += 4 * w.xs_pair_stride * (size_t)T;
  w.xs_sums = o; o += 4 * w.xs_sum_stride * (size_t)T;
  w.h_pong = o; o += n_layers > 0 ? up256(4 * H) : 0;
  // stacks: the routing accumulators of the two layer parities
  w.acc = o; o += n_layers > 0 ? up256(2 * 8 * acc_doubles(L->n_experts)) : 0;
  // token batches: per-pair down outputs and the expert groups
  const size_t P = (size_t)T * K;
  const bool batch = T > 1;
  w.y_routed = o; o += batch ? up256(4 * P * H) : 0;
  w.g_count = o; o += batch ? 256 : 0;
  w.g_expert = o; o += batch ? up256(4 * (P + 1)) : 0;
  w.g_start = o; o += batch ? up256(4 * (P + 2)) : 0;
  w.g_pair = o; o += batch ? up256(4 * P) : 0;
  w.ids = o; o += up256(4 * (size_t)kMaxK);  // cache slots of the routed experts (tier path)
  w.rec_src = o; o += up256(16 * (size_t)kMaxK);  // their record addresses and fill targets (tier)
  // linear-attention blocks of a stack: projections, o, the block's output
  // and the down/combine launch's constant entry
  const bool gdn = gdn_D > 0;
  w.gdn_proj = o; o += gdn ? up256(4 * (3 * (size_t)gdn_D + 2 * (size_t)gdn_heads)) : 0;
  w.gdn_o = o; o += gdn ? up256(4 * (size_t)gdn_D) : 0;
  w.gdn_h = o; o += gdn ? up256(4 * H) : 0;
  w.gdn_const = o; o += gdn ? 256 : 0;
  w.total = o;
  return w;
}

int check_bits(int b, const char *what) {
  if (b != 4 && b != 2) return fail(MOE_EUNSUPPORTED, "%s = %d: only 4 and 2 are built", what, b);
  return MOE_OK;
}

int check_dtype(int d, const char *what) {
  if (d != MOE_F32 && d != MOE_BF16) return fail(MOE_EUNSUPPORTED, "%s = %d: not MOE_F32/MOE_BF16", what, d);
  return MOE_OK;
}

// shapes, flags and weight pointers of a layer
int check_layer(const moe_layer_t *L) {
  if (!L) return fail(MOE_EINVAL, "layer is NULL");
  if (L->group != kGroup) return fail(MOE_EUNSUPPORTED, "group = %d: only 64 is built", L->group);
  int st;
  if ((st = check_bits(L->bits_routed, "bits_routed")) != MOE_OK) return st;
  if ((st = check_bits(L->bits_shared, "bits_shared")) != MOE_OK) return st;
  if ((st = check_dtype(L->router_dtype, "router_dtype")) != MOE_OK) return st;
  if ((st = check_dtype(L->gate_dtype, "gate_dtype")) != MOE_OK) return st;
  if (!dim_ok(L->hidden)) return fail(MOE_EINVAL, "hidden = %d: need a multiple of 64 in [64, 8192]", L->hidden);
  if (!dim_ok(L->inter)) return fail(MOE_EINVAL, "inter = %d: need a multiple of 64 in [64, 8192]", L->inter);
  if (L->top_k < 1 || L->top_k > kMaxK) return fail(MOE_EINVAL, "top_k = %d: need 1..8", L->top_k);
  if (L->n_experts < L->top_k || L->n_experts > kMaxE)
    return fail(MOE_EINVAL, "n_experts = %d: need top_k..1024", L->n_experts);
  if (L->renorm_topk != 0 && L->renorm_topk != 1) return fail(MOE_EINVAL, "renorm_topk must be 0 or 1");
  if (!L->router || !L->shared_gate || !L->experts || !L->shared_expert)
    return fail(MOE_EINVAL, "a weight pointer of the layer is NULL");
  if (!aligned(L->router, 16) || !aligned(L->shared_gate, 16) || !aligned(L->router_tiles, 16))
    return fail(MOE_EALIGN, "router, router_tiles and shared_gate must be 16-byte aligned");
  if (!aligned(L->experts, 256) || !aligned(L->shared_expert, 256) || L->expert_stride % 256)
    return fail(MOE_EALIGN, "expert records and expert_stride must be 256-byte aligned");
  const size_t rb = moe_expert_bytes(L->hidden, L->inter, L->bits_routed, L->group);
  if (L->expert_stride < rb)
    return fail(MOE_EINVAL, "expert_stride %zu < record size %zu", L->expert_stride, rb);
  return MOE_OK;
}

int check_tokens(int T) {
  if (T < 1 || T > kMaxTokens) return fail(MOE_EINVAL, "n_tokens = %d: need 1..64", T);
  return MOE_OK;
}

int check_vec(const void *p, const char *what) {
  if (!p) return fail(MOE_EINVAL, "%s is NULL", what);
  if (!aligned(p, 16)) return fail(MOE_EALIGN, "%s must be 16-byte aligned", what);
  return MOE_OK;
}

int check_ws(void *ws, size_t have, size_t need) {
  if (!ws) return fail(MOE_EWORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned(ws, 256)) return fail(MOE_EALIGN, "workspace must be 256-byte aligned");
  if (have < need) return fail(MOE_EWORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
  return MOE_OK;
}

RecOffsets offsets_of(int H, int I, int bits) { return record_offsets(H, I, bits); }

HeadParams head_params(const moe_layer_t *L, int T) {
  HeadParams h;
  memset(&h, 0, sizeof h);
  h.H = L->hidden;
  h.I = L->inter;
  h.E = L->n_experts;
  h.T = T;
  h.router_dtype = L->router_dtype;
  h.router = L->router;
  h.gate_dtype = L->gate_dtype;
  h.gvec = L->shared_gate;
  h.bits_shared = L->bits_shared;
  h.shared_rec = static_cast<const uint8_t *>(L->shared_expert);
  h.soff = offsets_of(L->hidden, L->inter, L->bits_shared);
  return h;
}

#define MOE_TRY_HIP(expr, what)              \
  do {                                       \
    hipError_t e_ = (expr);                  \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

// one token through one layer (x given, or x = rmsnorm(h_in + upd) when
// xsrc == XS_NORM), writes h_out, idx[K], w[K]
int layer_token(const moe_layer_t *L, int xsrc, const void *x, const float *h_in,
                const uint16_t *upd, const float *h_res, float *h_out, int32_t *idx, float *w,
                uint8_t *ws, const WsLayout &wl, hipStream_t s) {
  float *logits = reinterpret_cast<float *>(ws + wl.logits);
  float *sigma = reinterpret_cast<float *>(ws + wl.sigma);
  float *h_routed = reinterpret_cast<float *>(ws + wl.h_routed);
  float *h_shared = reinterpret_cast<float *>(ws + wl.h_shared);
  float *y_shared = reinterpret_cast<float *>(ws + wl.y_shared);
  float *x_stage = reinterpret_cast<float *>(ws + wl.x_stage);
  float *hres_stage = reinterpret_cast<float *>(ws + wl.hres_stage);
  // each gate/up workgroup stages x from x itself: reading the input is
  // faster than waiting for a staging buffer the router kernel has just
  // written (data written by the previous kernel come from memory)

  // K1
  HeadParams hp = head_params(L, 1);
  hp.xsrc = xsrc;
  hp.x = x;
  hp.h_in = h_in;
  hp.upd = upd;
  hp.logits = logits;
  hp.sigma = sigma;
  if (xsrc == XS_NORM) {
    hp.x_out = x_stage;
    hp.hres_out = hres_stage;
  }
  hp.h_shared = h_shared;
  // the shared expert's gate/up runs with the routed ones (K2) when both have
  // the same width; otherwise here (K1)
  const bool same_width = L->bits_shared == L->bits_routed;
  hp.n_shared_waves = same_width ? 0 : 1;  // launcher sizes it
  hp.bits_routed = L->bits_routed;
  MOE_TRY_HIP(timed(s, MOE_KERNEL_HEAD, [&] { return launch_head(hp, s); }), "router/shared launch");

  // K2
  GateUpParams gp;
  memset(&gp, 0, sizeof gp);
  gp.H = L->hidden;
  gp.I = L->inter;
  gp.E = L->n_experts;
  gp.K = L->top_k;
  gp.renorm = L->renorm_topk;
  gp.bits = L->bits_routed;
  gp.experts = static_cast<const uint8_t *>(L->experts);
  gp.stride = L->expert_stride;
  gp.shared_rec = static_cast<const uint8_t *>(L->shared_expert);
  gp.shared_ok = L->bits_shared == L->bits_routed;
  gp.off = offsets_of(L->hidden, L->inter, L->bits_routed);
  gp.soff = offsets_of(L->hidden, L->inter, L->bits_shared);
  gp.ids = nullptr;
  gp.n = L->top_k;
  gp.logits = logits;
  gp.idx_out = idx;
  gp.w_out = w;
  gp.xsrc = xsrc == XS_BF16 ? XS_BF16 : XS_F32;
  gp.x = xsrc == XS_NORM ? static_cast<const void *>(x_stage) : x;
  gp.h_out = h_routed;
  gp.with_shared = same_width;
  gp.h_shared_out = h_shared;
  MOE_TRY_HIP(timed(s, MOE_KERNEL_GATEUP, [&] { return launch_gateup(gp, s); }), "routed gate/up launch");

  // K3 (+ the shared down in its own launch when its width differs)
  DownParams dp;
  memset(&dp, 0, sizeof dp);
  dp.H = L->hidden;
  dp.I = L->inter;
  dp.E = L->n_experts;
  dp.experts = gp.experts;
  dp.stride = gp.stride;
  dp.shared_rec = gp.shared_rec;
  dp.off = gp.off;
  dp.soff = gp.soff;
  dp.shared_ok = 1;
  const bool same = same_width;
  if (!same) {
    // shared expert of another width: its down projection runs on its own
    // (a null id list selects the shared record) and K3 adds sigma * y_shared
    DownParams sp = dp;
    sp.combine = 0;
    sp.bits_r = L->bits_shared;
    sp.ids = nullptr;
    sp.n = 1;
    sp.h = h_shared;
    sp.y = y_shared;
    MOE_TRY_HIP(timed(s, MOE_KERNEL_DOWN_Y, [&] { return launch_down(sp, s); }), "shared down launch");
  }
  dp.combine = 1;
  dp.bits_r = L->bits_routed;
  dp.bits_s = L->bits_shared;
  dp.idx = idx;
  dp.w = w;
  dp.K = L->top_k;
  dp.sigma = sigma;
  dp.h_routed = h_routed;
  dp.h_shared = same ? h_shared : nullptr;
  dp.y = same ? nullptr : y_shared;
  dp.h_res = xsrc == XS_NORM ? hres_stage : h_res;
  dp.out = h_out;
  MOE_TRY_HIP(timed(s, MOE_KERNEL_DOWN, [&] { return launch_down(dp, s); }), "down/combine launch");
  return MOE_OK;
}

int expert_forward(const moe_layer_t *L, int bits, moe_dtype x_dtype, const void *x,
                   const int32_t *ids, int n, float *y, float *h, void *ws, size_t ws_bytes,
                   void *stream) {
  int st;
  if ((st = check_layer(L)) != MOE_OK) return st;
  if (L->bits_routed != bits)
    return fail(MOE_EUNSUPPORTED, "layer bits_routed = %d but this entry point is %d-bit", L->bits_routed, bits);
  if ((st = check_dtype(x_dtype, "x_dtype")) != MOE_OK) return st;
  if ((st = check_vec(x, "x")) != MOE_OK) return st;
  if ((st = check_vec(y, "y")) != MOE_OK) return st;
  if (!ids) return fail(MOE_EINVAL, "expert_ids is NULL");
  if (!aligned(ids, 4)) return fail(MOE_EALIGN, "expert_ids must be 4-byte aligned");
  if (n < 1 || n > kMaxTokens) return fail(MOE_EINVAL, "n = %d: need 1..64", n);
  if (h && !aligned(h, 16)) return fail(MOE_EALIGN, "h must be 16-byte aligned");
  const WsLayout wl = ws_layout(L, 1, 0);
  if ((st = check_ws(ws, ws_bytes, wl.total)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t *wsb = static_cast<uint8_t *>(ws);
  float *hbuf = h ? h : reinterpret_cast<float *>(wsb + wl.h_routed);

  GateUpParams gp;
  memset(&gp, 0, sizeof gp);
  gp.H = L->hidden;
  gp.I = L->inter;
  gp.E = L->n_experts;
  gp.K = L->top_k;
  gp.bits = bits;
  gp.experts = static_cast<const uint8_t *>(L->experts);
  gp.stride = L->expert_stride;
  gp.shared_rec = static_cast<const uint8_t *>(L->shared_expert);
  gp.shared_ok = L->bits_shared == bits;
  gp.off = offsets_of(L->hidden, L->inter, bits);
  gp.soff = offsets_of(L->hidden, L->inter, L->bits_shared);
  gp.ids = ids;
  gp.n = n;
  gp.xsrc = x_dtype == MOE_BF16 ? XS_BF16 : XS_F32;
  gp.x = x;
  gp.h_out = hbuf;
  MOE_TRY_HIP(timed(s, MOE_KERNEL_GATEUP, [&] { return launch_gateup(gp, s); }), "gate/up launch");

  DownParams dp;
  memset(&dp, 0, sizeof dp);
  dp.H = L->hidden;
  dp.I = L->inter;
  dp.E = L->n_experts;
  dp.bits_r = bits;
  dp.bits_s = L->bits_shared;
  dp.experts = gp.experts;
  dp.stride = gp.stride;
  dp.shared_rec = gp.shared_rec;
  dp.off = gp.off;
  dp.soff = gp.soff;
  dp.combine = 0;
  dp.ids = ids;
  dp.n = n;
  dp.h = hbuf;
  dp.y = y;
  dp.shared_ok = gp.shared_ok;
  MOE_TRY_HIP(timed(s, MOE_KERNEL_DOWN_Y, [&] { return launch_down(dp, s); }), "down launch");
  return MOE_OK;
}

}  // namespace

namespace moe_impl {
RecOffsets record_offsets(int hidden, int inter, int bits) {
  RecOffsets r;
  const size_t gc = (size_t)inter * hidden * bits / 8;
  const size_t dc = (size_t)hidden * inter * bits / 8;
  const size_t gs = (size_t)inter * (hidden / kGroup) * 4;
  const size_t ds = (size_t)hidden * (inter / kGroup) * 4;
  r.gate_codes = 0;
  r.up_codes = r.gate_codes + up256(gc);
  r.down_codes = r.up_codes + up256(gc);
  r.gate_sb = r.down_codes + up256(dc);
  r.up_sb = r.gate_sb + up256(gs);
  r.down_sb = r.up_sb + up256(gs);
  r.total = r.down_sb + up256(ds);
  return r;
}
}  // namespace moe_impl

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

const char *moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported configuration";
    case MOE_EALIGN: return "misaligned pointer or stride";
    case MOE_EWORKSPACE: return "workspace missing or too small";
    case MOE_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char *moe_last_error(void) { return g_err; }

int moe_abi_version(void) { return 2; }

size_t moe_qmatrix_bytes(int rows, int cols, int bits, int group) {
  if (group != kGroup || (bits != 4 && bits != 2) || rows < 1 || cols < kGroup || cols % kGroup) return 0;
  return up256((size_t)rows * cols * bits / 8) + up256((size_t)rows * (cols / kGroup) * 4);
}

size_t moe_expert_bytes(int hidden, int inter, int bits, int group) {
  if (group != kGroup || (bits != 4 && bits != 2) || !dim_ok(hidden) || !dim_ok(inter)) return 0;
  return record_offsets(hidden, inter, bits).total;
}

int moe_expert_offsets(int hidden, int inter, int bits, int group, size_t out[6]) {
  if (!out) return fail(MOE_EINVAL, "out is NULL");
  if (moe_expert_bytes(hidden, inter, bits, group) == 0)
    return fail(MOE_EINVAL, "invalid record shape (%d, %d, %d bits, group %d)", hidden, inter, bits, group);
  const RecOffsets r = record_offsets(hidden, inter, bits);
  out[0] = r.gate_codes; out[1] = r.up_codes; out[2] = r.down_codes;
  out[3] = r.gate_sb; out[4] = r.up_sb; out[5] = r.down_sb;
  return MOE_OK;
}

size_t moe_layer_workspace_bytes(const moe_layer_t *L, int n_tokens) {
  if (!L || n_tokens < 1 || n_tokens > kMaxTokens) return 0;
  if (L->top_k < 1 || L->top_k > kMaxK || L->n_experts < 1 || !dim_ok(L->hidden) || !dim_ok(L->inter)) return 0;
  return ws_layout(L, n_tokens, 0).total;
}

size_t moe_stack_workspace_bytes(const moe_layer_t *L, int n_layers) {
  if (!L || n_layers < 1) return 0;
  if (L->top_k < 1 || L->top_k > kMaxK || L->n_experts < 1 || !dim_ok(L->hidden) || !dim_ok(L->inter)) return 0;
  return ws_layout(L, 1, n_layers).total;
}

int moe_route(const moe_layer_t *L, int n_tokens, moe_dtype x_dtype, const void *x,
              int32_t *topk_idx, float *topk_w, float *shared_sigma, float *logits,
              void *ws, size_t ws_bytes, void *stream) {
  int st;
  if ((st = check_layer(L)) != MOE_OK) return st;
  if ((st = check_tokens(n_tokens)) != MOE_OK) return st;
  if ((st = check_dtype(x_dtype, "x_dtype")) != MOE_OK) return st;
  if ((st = check_vec(x, "x")) != MOE_OK) return st;
  if (!topk_idx || !topk_w || !shared_sigma) return fail(MOE_EINVAL, "an output pointer is NULL");
  if (!aligned(topk_idx, 4) || !aligned(topk_w, 4) || !aligned(shared_sigma, 4))
    return fail(MOE_EALIGN, "outputs must be 4-byte aligned");
  // the top-K kernel reads the logits with 16-byte loads
  if (logits && !aligned(logits, 16)) return fail(MOE_EALIGN, "logits must be 16-byte aligned");
  const WsLayout wl = ws_layout(L, n_tokens, 0);
  if ((st = check_ws(ws, ws_bytes, wl.total)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t *wsb = static_cast<uint8_t *>(ws);
  float *lg = logits ? logits : reinterpret_cast<float *>(wsb + wl.logits);
  HeadParams hp = head_params(L, n_tokens);
  hp.xsrc = x_dtype == MOE_BF16 ? XS_BF16 : XS_F32;
  hp.x = x;
  hp.logits = lg;
  hp.sigma = shared_sigma;
  hp.n_shared_waves = 0;
  MOE_TRY_HIP(timed(s, MOE_KERNEL_HEAD, [&] { return launch_head(hp, s); }), "router launch");
  TopkParams tp;
  tp.logits = lg;
  tp.T = n_tokens;
  tp.E = L->n_experts;
  tp.K = L->top_k;
  tp.renorm = L->renorm_topk;
  tp.idx = topk_idx;
  tp.w = topk_w;
  MOE_TRY_HIP(timed(s, MOE_KERNEL_TOPK, [&] { return launch_topk(tp, s); }), "top-K launch");
  return MOE_OK;
}

int moe_expert_forward_q4(const moe_layer_t *L, moe_dtype x_dtype, const void *x,
                          const int32_t *expert_ids, int n, float *y, float *h, void *ws,
                          size_t ws_bytes, void *stream) {
  return expert_forward(L, 4, x_dtype, x, expert_ids, n, y, h, ws, ws_bytes, stream);
}

int moe_expert_forward_q2(const moe_layer_t *L, moe_dtype x_dtype, const void *x,
                          const int32_t *expert_ids, int n, float *y, float *h, void *ws,
                          size_t ws_bytes, void *stream) {
  return expert_forward(L, 2, x_dtype, x, expert_ids, n, y, h, ws, ws_bytes, stream);
}

int moe_combine(int hidden, int n_routed, const float *h_res, const float *y, const float *w,
                const float *y_shared, const float *shared_sigma, float *h_out, void *stream) {
  if (hidden < 1 || hidden > kMaxDim) return fail(MOE_EINVAL, "hidden = %d out of range", hidden);
  if (n_routed < 0 || n_routed > kMaxK * kMaxTokens) return fail(MOE_EINVAL, "n_routed = %d out of range", n_routed);
  int st;
  if ((st = check_vec(h_res, "h_res")) != MOE_OK) return st;
  if ((st = check_vec(y_shared, "y_shared")) != MOE_OK) return st;
  if ((st = check_vec(h_out, "h_out")) != MOE_OK) return st;
  if (n_routed > 0) {
    if ((st = check_vec(y, "y")) != MOE_OK) return st;
    if (!w) return fail(MOE_EINVAL, "w is NULL");
  }
  if (!shared_sigma) return fail(MOE_EINVAL, "shared_sigma is NULL");
  CombineParams p;
  p.H = hidden;
  p.K = n_routed;
  p.h_res = h_res;
  p.y = y;
  p.w = w;
  p.y_shared = y_shared;
  p.sigma = shared_sigma;
  p.out = h_out;
  hipStream_t s = static_cast<hipStream_t>(stream);
  MOE_TRY_HIP(timed(s, MOE_KERNEL_COMBINE, [&] { return launch_combine(p, s); }), "combine launch");
  return MOE_OK;
}

// T > 1 tokens through one layer: router rows for every token, then the
// top-K of every token and the (token, expert) pairs grouped by expert, so
// that gate/up and down read each distinct expert's weights once for all of
// its tokens; then the per-token combine
int layer_batch(const moe_layer_t *L, int T, int xsrc, const void *x, const float *h_res,
                float *h_out, int32_t *idx, float *w, uint8_t *ws, const WsLayout &wl,
                hipStream_t s) {
  float *logits = reinterpret_cast<float *>(ws + wl.logits);
  float *sigma = reinterpret_cast<float *>(ws + wl.sigma);
  uint32_t *xs_pairs = xsrc == XS_BF16 ? reinterpret_cast<uint32_t *>(ws + wl.xs_pairs) : nullptr;
  float *xs_sums = xsrc == XS_BF16 ? reinterpret_cast<float *>(ws + wl.xs_sums) : nullptr;
  int32_t *g_count = reinterpret_cast<int32_t *>(ws + wl.g_count);
  int32_t *g_expert = reinterpret_cast<int32_t *>(ws + wl.g_expert);
  int32_t *g_start = reinterpret_cast<int32_t *>(ws + wl.g_start);
  int32_t *g_pair = reinterpret_cast<int32_t *>(ws + wl.g_pair);

  HeadParams hp = head_params(L, T);
  hp.xsrc = xsrc;
  hp.x = x;
  hp.logits = logits;
  hp.sigma = sigma;
  hp.n_shared_waves = 0;
  hp.bits_routed = L->bits_routed;
  hp.xs_pairs = xs_pairs;
  hp.xs_sums = xs_sums;
  hp.xs_pair_stride = (int)wl.xs_pair_stride;
  hp.xs_sum_stride = (int)wl.xs_sum_stride;
  MOE_TRY_HIP(timed(s, MOE_KERNEL_HEAD, [&] { return launch_head(hp, s); }), "router launch");

  // every token's selection in a workgroup of its own, then the grouping in
  // one workgroup (a single workgroup selecting for every token took 12.8 us
  // of the 16-token q4 call)
  TopkParams tp;
  tp.logits = logits;
  tp.T = T;
  tp.E = L->n_experts;
  tp.K = L->top_k;
  tp.renorm = L->renorm_topk;
  tp.idx = idx;
  tp.w = w;
  MOE_TRY_HIP(timed(s, MOE_KERNEL_TOPK, [&] { return launch_topk(tp, s); }), "top-K launch");
  RouteGroupParams rg;
  rg.logits = logits;
  rg.T = T;
  rg.E = L->n_experts;
  rg.K = L->top_k;
  rg.renorm = L->renorm_topk;
  rg.selected = 1;
  rg.idx = idx;
  rg.w = w;
  rg.g_count = g_count;
  rg.g_expert = g_expert;
  rg.g_start = g_start;
  rg.g_pair = g_pair;
  // small batches: the grouped gate/up kernel groups the pairs itself
  const bool group_in_kernel = T * L->top_k <= kGroupInKernel;
  if (!group_in_kernel)
    MOE_TRY_HIP(timed(s, MOE_KERNEL_TOPK, [&] { return launch_route_group(rg, s); }), "grouping launch");

  GroupedParams gp;
  memset(&gp, 0, sizeof gp);
  gp.H = L->hidden;
  gp.I = L->inter;
  gp.E = L->n_experts;
  gp.K = L->top_k;
  gp.T = T;
  gp.experts = static_cast<const uint8_t *>(L->experts);
  gp.stride = L->expert_stride;
  gp.shared_rec = static_cast<const uint8_t *>(L->shared_expert);
  gp.off = offsets_of(L->hidden, L->inter, L->bits_routed);
  gp.soff = offsets_of(L->hidden, L->inter, L->bits_shared);
  gp.g_count = g_count;
  gp.g_expert = g_expert;
  gp.g_start = g_start;
  gp.g_pair = g_pair;
  gp.xsrc = xsrc;
  gp.x = x;
  gp.xs_pairs = xs_pairs;
  gp.xs_sums = xs_sums;
  gp.xs_pair_stride = (int)wl.xs_pair_stride;
  gp.xs_sum_stride = (int)wl.xs_sum_stride;
  gp.h_routed = reinterpret_cast<float *>(ws + wl.h_routed);
  gp.h_shared = reinterpret_cast<float *>(ws + wl.h_shared);
  gp.y_routed = reinterpret_cast<float *>(ws + wl.y_routed);
  gp.y_shared = reinterpret_cast<float *>(ws + wl.y_shared);
  const bool same = L->bits_shared == L->bits_routed;
  // routed groups (and the shared one when it has the same width)
  GroupedParams gr = gp;
  gr.bits = L->bits_routed;
  gr.do_routed = 1;
  gr.do_shared = same;
  GroupedParams gr_gu = gr;  // the gate/up launch, which may group the pairs
  if (group_in_kernel) gr_gu.group_idx = idx;
  GroupedParams gs = gp;  // the shared expert alone, at its own width
  gs.bits = L->bits_shared;
  gs.do_routed = 0;
  gs.do_shared = 1;
  gs.xs_pairs = nullptr;  // x was staged for the routed width
  gs.xs_sums = nullptr;
  MOE_TRY_HIP(timed(s, MOE_KERNEL_GATEUP, [&] { return launch_gateup_grouped(gr_gu, s); }), "grouped gate/up launch");
  if (!same)
    MOE_TRY_HIP(timed(s, MOE_KERNEL_GATEUP, [&] { return launch_gateup_grouped(gs, s); }), "shared gate/up launch");
  MOE_TRY_HIP(timed(s, MOE_KERNEL_DOWN_Y, [&] { return launch_down_grouped(gr, s); }), "grouped down launch");
  if (!same)
    MOE_TRY_HIP(timed(s, MOE_KERNEL_DOWN_Y, [&] { return launch_down_grouped(gs, s); }), "shared down launch");

  CombineTokensParams cp;
  cp.H = L->hidden;
  cp.K = L->top_k;
  cp.T = T;
  cp.h_res = h_res;
  cp.y_routed = gp.y_routed;
  cp.w = w;
  cp.y_shared = gp.y_shared;
  cp.sigma = sigma;
  cp.out = h_out;
  MOE_TRY_HIP(timed(s, MOE_KERNEL_COMBINE, [&] { return launch_combine_tokens(cp, s); }), "combine launch");
  return MOE_OK;
}

// the arguments of a layer decode other than its workspace
static int check_decode_args(const moe_layer_t *L, int n_tokens, moe_dtype x_dtype, const void *x,
                             const float *h_res, const float *h_out, const int32_t *topk_idx,
                             const float *topk_w) {
  int st;
  if ((st = check_layer(L)) != MOE_OK) return st;
  if ((st = check_tokens(n_tokens)) != MOE_OK) return st;
  if ((st = check_dtype(x_dtype, "x_dtype")) != MOE_OK) return st;
  if ((st = check_vec(x, "x")) != MOE_OK) return st;
  if ((st = check_vec(h_res, "h_res")) != MOE_OK) return st;
  if ((st = check_vec(h_out, "h_out")) != MOE_OK) return st;
  if (h_out == h_res) return fail(MOE_EINVAL, "h_out may not alias h_res");
  if (!topk_idx || !topk_w) return fail(MOE_EINVAL, "topk_idx / topk_w is NULL");
  if (!aligned(topk_idx, 4) || !aligned(topk_w, 4)) return fail(MOE_EALIGN, "topk outputs must be 4-byte aligned");
  return MOE_OK;
}

int moe_layer_decode(const moe_layer_t *L, int n_tokens, moe_dtype x_dtype, const void *x,
                     const float *h_res, float *h_out, int32_t *topk_idx, float *topk_w,
                     void *ws, size_t ws_bytes, void *stream) {
  int st;
  if ((st = check_decode_args(L, n_tokens, x_dtype, x, h_res, h_out, topk_idx, topk_w)) != MOE_OK)
    return st;
  const WsLayout wl = ws_layout(L, n_tokens, 0);
  if ((st = check_ws(ws, ws_bytes, wl.total)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int xsrc = x_dtype == MOE_BF16 ? XS_BF16 : XS_F32;
  const size_t xes = x_dtype == MOE_BF16 ? 2 : 4;
  (void)xes;
  if (n_tokens > 1)
    return layer_batch(L, n_tokens, xsrc, x, h_res, h_out, topk_idx, topk_w,
                       static_cast<uint8_t *>(ws), wl, s);
  return layer_token(L, xsrc, x, nullptr, nullptr, h_res, h_out, topk_idx, topk_w,
                     static_cast<uint8_t *>(ws), wl, s);
}

int moe_layer_decode_noalloc(const moe_layer_t *L, int n_tokens, moe_dtype x_dtype,
                             const void *x, const float *h_res, float *h_out,
                             int32_t *topk_idx, float *topk_w, void *stream) {
  int st;
  if ((st = check_decode_args(L, n_tokens, x_dtype, x, h_res, h_out, topk_idx, topk_w)) != MOE_OK)
    return st;
  const size_t need = ws_layout(L, n_tokens, 0).total;
  if (need > kNoAllocScratchBytes)
    return fail(MOE_EWORKSPACE, "this layer and token count need %zu bytes of workspace; the "
                "library's own scratch holds %zu (use moe_layer_decode with a workspace)",
                need, kNoAllocScratchBytes);
  void *scratch = nullptr;
  MOE_TRY_HIP(noalloc_scratch(&scratch), "looking up the scratch array");
  return moe_layer_decode(L, n_tokens, x_dtype, x, h_res, h_out, topk_idx, topk_w, scratch,
                          kNoAllocScratchBytes, stream);
}

int moe_layer_ws_view(const moe_layer_t *L, int n_tokens, void *ws, size_t ws_bytes,
                      moe_ws_view *view) {
  int st;
  if ((st = check_layer(L)) != MOE_OK) return st;
  if ((st = check_tokens(n_tokens)) != MOE_OK) return st;
  if (!view) return fail(MOE_EINVAL, "view is NULL");
  const WsLayout wl = ws_layout(L, n_tokens, 0);
  if ((st = check_ws(ws, ws_bytes, wl.total)) != MOE_OK) return st;
  uint8_t *b = static_cast<uint8_t *>(ws);
  view->logits = reinterpret_cast<float *>(b + wl.logits);
  view->sigma = reinterpret_cast<float *>(b + wl.sigma);
  view->h_routed = reinterpret_cast<float *>(b + wl.h_routed);
  view->h_shared = reinterpret_cast<float *>(b + wl.h_shared);
  return MOE_OK;
}

static int stack_run(const moe_layer_t *layers, int n_layers, const uint16_t *updates, float *h,
                     int32_t *idx_log, float *w_log, uint8_t *ws, const WsLayout &wl, hipStream_t s);

// whether a stack runs with two kernels per layer (stack_run): a shared expert
// of the routed width (the gate/up launch takes it), and combine launches whose
// workgroups cover row tiles the routing partials can take; otherwise the
// layers run as router, gate/up and down/combine kernels.  Stacks with
// linear-attention blocks keep the router kernel: forming the partials in the
// block's output projection (rows of 8192 codes, two rounds of workgroups)
// cost more than the router launch it saves (60-layer stack: 49.3 against
// 48.4 us per layer).
static bool stack_two_kernels(const moe_layer_t *layers) {
  const moe_layer_t &L = layers[0];
  return L.bits_shared == L.bits_routed &&
         combine_takes_partials(L.hidden, L.inter, L.bits_routed, L.top_k + 1);
}

int moe_stack_decode(const moe_layer_t *layers, int n_layers, const uint16_t *updates_bf16,
                     float *h, int32_t *idx_log, float *w_log, void *ws, size_t ws_bytes,
                     void *stream) {
  if (!layers) return fail(MOE_EINVAL, "layers is NULL");
  if (n_layers < 1) return fail(MOE_EINVAL, "n_layers = %d", n_layers);
  int st;
  for (int l = 0; l < n_layers; ++l) {
    if ((st = check_layer(&layers[l])) != MOE_OK) return st;
    const moe_layer_t &a = layers[0], &b = layers[l];
    if (a.hidden != b.hidden || a.inter != b.inter || a.n_experts != b.n_experts ||
        a.top_k != b.top_k || a.bits_routed != b.bits_routed || a.bits_shared != b.bits_shared ||
        a.router_dtype != b.router_dtype || a.gate_dtype != b.gate_dtype)
      return fail(MOE_EINVAL, "layer %d differs in shape or format from layer 0", l);
  }
  if ((st = check_vec(h, "h")) != MOE_OK) return st;
  if (updates_bf16 && !aligned(updates_bf16, 16)) return fail(MOE_EALIGN, "updates must be 16-byte aligned");
  if (!idx_log || !w_log) return fail(MOE_EINVAL, "idx_log / w_log is NULL");
  if (!aligned(idx_log, 4) || !aligned(w_log, 4)) return fail(MOE_EALIGN, "logs must be 4-byte aligned");
  const moe_layer_t *L = &layers[0];
  const WsLayout wl = ws_layout(L, 1, n_layers);
  if ((st = check_ws(ws, ws_bytes, wl.total)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t *wsb = static_cast<uint8_t *>(ws);
  if (stack_two_kernels(layers))
    return stack_run(layers, n_layers, updates_bf16, h, idx_log, w_log, wsb, wl, s);
  // otherwise (a shared expert of another width keeps its gate/up in the
  // router kernel): three kernels per layer
  float *pong = reinterpret_cast<float *>(wsb + wl.h_pong);
  const size_t H = L->hidden, K = L->top_k;
  float *cur = h, *nxt = pong;
  for (int l = 0; l < n_layers; ++l) {
    const uint16_t *u = updates_bf16 ? updates_bf16 + (size_t)l * H : nullptr;
    st = layer_token(&layers[l], XS_NORM, nullptr, cur, u, nullptr, nxt, idx_log + l * K,
                     w_log + l * K, wsb, wl, s);
    if (st != MOE_OK) return st;
    float *t = cur;
    cur = nxt;
    nxt = t;
  }
  if (cur != h)
    MOE_TRY_HIP(timed(s, MOE_KERNEL_OTHER, [&] { return launch_copy_f32(h, cur, L->hidden, s); }), "copy launch");
  return MOE_OK;
}

int moe_router_tile(const void *router, int n_experts, int hidden, moe_dtype router_dtype,
                    void *out, void *stream) {
  int st;
  if ((st = check_dtype(router_dtype, "router_dtype")) != MOE_OK) return st;
  if (n_experts < 1 || n_experts > kMaxE) return fail(MOE_EINVAL, "n_experts = %d: need 1..1024", n_experts);
  if (!dim_ok(hidden)) return fail(MOE_EINVAL, "hidden = %d: need a multiple of 64 in [64, 8192]", hidden);
  if ((st = check_vec(router, "router")) != MOE_OK) return st;
  if ((st = check_vec(out, "out")) != MOE_OK) return st;
  const size_t esz = router_dtype == MOE_BF16 ? 2 : 4;
  const size_t bytes = (size_t)n_experts * hidden * esz;
  const uintptr_t a = reinterpret_cast<uintptr_t>(router), b = reinterpret_cast<uintptr_t>(out);
  if (a < b + bytes && b < a + bytes) return fail(MOE_EINVAL, "out overlaps router");
  hipStream_t s = static_cast<hipStream_t>(stream);
  MOE_TRY_HIP(timed(s, MOE_KERNEL_OTHER, [&] { return launch_router_tile(router, n_experts, hidden, (int)esz, out, s); }),
              "router tile launch");
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// stacks with linear-attention blocks
// ---------------------------------------------------------------------------
static int check_gdn(const moe_layer_t *L, const moe_gdn_layer_t *g, int l) {
  if (g->n_heads < 1 || (g->d_head != 16 && g->d_head != 32 && g->d_head != 64 && g->d_head != 128 &&
                         g->d_head != 256))
    return fail(MOE_EUNSUPPORTED, "layer %d: linear attention needs d_head in {16, 32, 64, 128, 256}, "
                "n_heads >= 1 (got %d, %d)", l, g->d_head, g->n_heads);
  const int D = g->n_heads * g->d_head;
  if (!dim_ok(D)) return fail(MOE_EINVAL, "layer %d: n_heads * d_head = %d: need a multiple of 64 in [64, 8192]", l, D);
  if (2 * g->n_heads > D) return fail(MOE_EINVAL, "layer %d: 2 n_heads exceeds the gate rows", l);
  int st;
  if ((st = check_bits(g->bits, "linear-attention bits")) != MOE_OK) return st;
  if (!g->rec_qko || !g->rec_vab) return fail(MOE_EINVAL, "layer %d: a projection record is NULL", l);
  if (!aligned(g->rec_qko, 256) || !aligned(g->rec_vab, 256))
    return fail(MOE_EALIGN, "layer %d: projection records must be 256-byte aligned", l);
  if (!aligned(g->state, 16)) return fail(MOE_EALIGN, "layer %d: state must be 16-byte aligned", l);
  (void)L;
  return MOE_OK;
}

static void gdn_extent(const moe_gdn_layer_t *gdn, int n_layers, int &D, int &heads) {
  D = heads = 0;
  for (int l = 0; gdn && l < n_layers; ++l) {
    if (!gdn[l].state) continue;
    if (gdn[l].n_heads * gdn[l].d_head > D) D = gdn[l].n_heads * gdn[l].d_head;
    if (gdn[l].n_heads > heads) heads = gdn[l].n_heads;
  }
}

// x = RMSNorm(h); projections; the delta-rule step on the layer's state;
// h_out = h + W_o o (the down/combine kernel with W_o as its one expert)
static int gdn_block(const moe_layer_t *L, const moe_gdn_layer_t *g, const float *h, float *h_out,
                     uint8_t *ws, const WsLayout &wl, hipStream_t s) {
  const int D = g->n_heads * g->d_head;
  float *proj = reinterpret_cast<float *>(ws + wl.gdn_proj);
  float *o = reinterpret_cast<float *>(ws + wl.gdn_o);
  int32_t *one_idx = reinterpret_cast<int32_t *>(ws + wl.gdn_const);
  float *one_w = reinterpret_cast<float *>(ws + wl.gdn_const) + 1;
  float *zero_sigma = reinterpret_cast<float *>(ws + wl.gdn_const) + 2;
  const RecOffsets off = offsets_of(L->hidden, D, g->bits);
  GdnInParams ip;
  memset(&ip, 0, sizeof ip);
  ip.H = L->hidden;
  ip.D = D;
  ip.n_heads = g->n_heads;
  ip.bits = g->bits;
  ip.h = h;
  ip.rec_qko = static_cast<const uint8_t *>(g->rec_qko);
  ip.rec_vab = static_cast<const uint8_t *>(g->rec_vab);
  ip.off = off;
  ip.proj = proj;
  ip.one_idx = one_idx;
  ip.one_w = one_w;
  ip.zero_sigma = zero_sigma;
  MOE_TRY_HIP(timed(s, MOE_KERNEL_GDN_IN, [&] { return launch_gdn_in(ip, s); }), "linear-attention projection launch");
  GdnParams gp;
  gp.n_sh = g->n_heads;
  gp.d_k = gp.d_v = g->d_head;
  gp.q = proj;
  gp.k = proj + D;
  gp.v = proj + 2 * D;
  gp.alpha = proj + 3 * D;
  gp.beta = proj + 3 * D + g->n_heads;
  gp.state = g->state;
  gp.out = o;
  gp.prep = 1;
  MOE_TRY_HIP(timed(s, MOE_KERNEL_GDN_STEP, [&] { return launch_gdn_step(gp, s); }), "delta-rule step launch");
  DownParams dp;
  memset(&dp, 0, sizeof dp);
  dp.H = L->hidden;
  dp.I = D;
  dp.E = 1;
  dp.bits_r = dp.bits_s = g->bits;
  dp.experts = static_cast<const uint8_t *>(g->rec_qko);
  dp.stride = off.total;
  dp.shared_rec = dp.experts;
  dp.off = dp.soff = off;
  dp.combine = 1;
  dp.idx = one_idx;
  dp.w = one_w;
  dp.K = 1;
  dp.fixed_first = 1;
  dp.sigma = zero_sigma;
  dp.h_routed = o;
  dp.h_shared = nullptr;
  dp.y = nullptr;
  dp.h_res = h;
  dp.out = h_out;
  dp.shared_ok = 1;
  MOE_TRY_HIP(timed(s, MOE_KERNEL_GDN_OUT, [&] { return launch_down(dp, s); }), "output projection launch");
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// stacks of same-width layers: two kernels per layer.  The down/combine
// kernel of layer l forms the next layer's input v = out + u_{l+1} and, for
// its rows, the partial router / gate dots and sum of squares of v
// (accumulated over workgroups in fp64, spread over kAccCopies copies); the
// gate/up kernel of layer l + 1 takes its routing and its x = v / rms(v) from
// those sums.  So no kernel runs between a layer's combine and the next
// layer's gate/up.  The first layer's sums come from k_partials (or from the
// output projection of its linear-attention block).
// ---------------------------------------------------------------------------
static int stack_gateup(const moe_layer_t *L, const float *v, const double *acc, double *acc_zero,
                        int32_t *idx, float *w, uint8_t *ws, const WsLayout &wl, hipStream_t s) {
  GateUpParams gp;
  memset(&gp, 0, sizeof gp);
  gp.H = L->hidden;
  gp.I = L->inter;
  gp.E = L->n_experts;
  gp.K = L->top_k;
  gp.renorm = L->renorm_topk;
  gp.bits = L->bits_routed;
  gp.experts = static_cast<const uint8_t *>(L->experts);
  gp.stride = L->expert_stride;
  gp.shared_rec = static_cast<const uint8_t *>(L->shared_expert);
  gp.shared_ok = 1;
  gp.off = offsets_of(L->hidden, L->inter, L->bits_routed);
  gp.soff = gp.off;
  gp.n = L->top_k;
  gp.idx_out = idx;
  gp.w_out = w;
  gp.xsrc = XS_F32;
  gp.x = v;
  gp.h_out = reinterpret_cast<float *>(ws + wl.h_routed);
  gp.with_shared = 1;
  gp.h_shared_out = reinterpret_cast<float *>(ws + wl.h_shared);
  gp.acc = acc;
  gp.acc_zero = acc_zero;
  gp.acc_zero_n = (int)acc_doubles(L->n_experts);
  gp.sigma_out = reinterpret_cast<float *>(ws + wl.sigma);
  MOE_TRY_HIP(timed(s, MOE_KERNEL_GATEUP, [&] { return launch_gateup(gp, s); }), "gate/up launch");
  return MOE_OK;
}

static int stack_down(const moe_layer_t *L, const float *v, float *out,
                      const int32_t *idx, const float *w, const moe_layer_t *next,
                      const uint16_t *u_next, double *acc_next, uint8_t *ws, const WsLayout &wl,
                      hipStream_t s) {
  DownParams dp;
  memset(&dp, 0, sizeof dp);
  dp.H = L->hidden;
  dp.I = L->inter;
  dp.E = L->n_experts;
  dp.experts = static_cast<const uint8_t *>(L->experts);
  dp.stride = L->expert_stride;
  dp.shared_rec = static_cast<const uint8_t *>(L->shared_expert);
  dp.off = dp.soff = offsets_of(L->hidden, L->inter, L->bits_routed);
  dp.shared_ok = 1;
  dp.combine = 1;
  dp.bits_r = dp.bits_s = L->bits_routed;
  dp.idx = idx;
  dp.w = w;
  dp.K = L->top_k;
  dp.sigma = reinterpret_cast<float *>(ws + wl.sigma);  // written by the gate/up launch
  dp.h_routed = reinterpret_cast<float *>(ws + wl.h_routed);
  dp.h_shared = reinterpret_cast<float *>(ws + wl.h_shared);
  dp.h_res = v;
  dp.out = out;
  if (next) {
    dp.nr_router = next->router;
    dp.nr_router_tiles = next->router_tiles;
    dp.nr_router_dtype = next->router_dtype;
    dp.nr_gate = next->shared_gate;
    dp.nr_gate_dtype = next->gate_dtype;
    dp.nr_upd = u_next;
    dp.nr_acc = acc_next;
    dp.nr_E = next->n_experts;
  }
  MOE_TRY_HIP(timed(s, MOE_KERNEL_DOWN, [&] { return launch_down(dp, s); }), "down/combine launch");
  return MOE_OK;
}

// layers share one width and have no linear-attention blocks
static int stack_run(const moe_layer_t *layers, int n_layers, const uint16_t *updates, float *h,
                     int32_t *idx_log, float *w_log, uint8_t *ws, const WsLayout &wl, hipStream_t s) {
  const moe_layer_t *L0 = &layers[0];
  const size_t H = L0->hidden, K = L0->top_k;
  const size_t nacc = acc_doubles(L0->n_experts);
  double *acc[2] = {reinterpret_cast<double *>(ws + wl.acc), reinterpret_cast<double *>(ws + wl.acc) + nacc};
  float *buf[2] = {h, reinterpret_cast<float *>(ws + wl.h_pong)};
  auto upd = [&](int l) { return updates ? updates + (size_t)l * H : nullptr; };
  MOE_TRY_HIP(timed(s, MOE_KERNEL_OTHER, [&] { return launch_zero(acc[0], 2 * nacc * sizeof(double), s); }),
              "accumulator zero launch");
  // layer 0's input v = h + u_0 and its routing sums.  The layers' outputs
  // alternate between h and the ping-pong buffer; v starts in h (k_partials
  // reads and writes each element in one thread, so in place is safe) when
  // the layer count is even, else in the other buffer, so that the last
  // layer's output lands in h and no copy follows.
  float *v = (n_layers % 2 == 0) ? buf[0] : buf[1];
  PartialsParams pp;
  pp.H = (int)H;
  pp.E = L0->n_experts;
  pp.h = h;
  pp.upd = upd(0);
  pp.v_out = v;
  pp.router = L0->router;
  pp.router_tiles = L0->router_tiles;
  pp.router_dtype = L0->router_dtype;
  pp.gate = L0->shared_gate;
  pp.gate_dtype = L0->gate_dtype;
  pp.acc = acc[0];
  MOE_TRY_HIP(timed(s, MOE_KERNEL_HEAD, [&] { return launch_partials(pp, s); }), "routing partials launch");
  int st;
  for (int l = 0; l < n_layers; ++l) {
    const moe_layer_t *Ll = &layers[l];
    int32_t *idx = idx_log + l * K;
    float *w = w_log + l * K;
    if ((st = stack_gateup(Ll, v, acc[l % 2], acc[(l + 1) % 2], idx, w, ws, wl, s)) != MOE_OK) return st;
    const bool last = l + 1 == n_layers;
    float *out = v == buf[0] ? buf[1] : buf[0];
    if ((st = stack_down(Ll, v, out, idx, w, last ? nullptr : &layers[l + 1], last ? nullptr : upd(l + 1),
                         last ? nullptr : acc[(l + 1) % 2], ws, wl, s)) != MOE_OK)
      return st;
    v = out;
  }
  if (v != h)
    MOE_TRY_HIP(timed(s, MOE_KERNEL_OTHER, [&] { return launch_copy_f32(h, v, L0->hidden, s); }), "copy launch");
  return MOE_OK;
}

size_t moe_stack_gdn_workspace_bytes(const moe_layer_t *L, const moe_gdn_layer_t *gdn, int n_layers) {
  if (!L || n_layers < 1) return 0;
  if (L->top_k < 1 || L->top_k > kMaxK || L->n_experts < 1 || !dim_ok(L->hidden) || !dim_ok(L->inter)) return 0;
  int D, heads;
  gdn_extent(gdn, n_layers, D, heads);
  return ws_layout(L, 1, n_layers, D, heads).total;
}

int moe_stack_decode_gdn(const moe_layer_t *layers, const moe_gdn_layer_t *gdn, int n_layers,
                         const uint16_t *updates_bf16, float *h, int32_t *idx_log, float *w_log,
                         void *ws, size_t ws_bytes, void *stream) {
  if (!layers || !gdn) return fail(MOE_EINVAL, "layers / gdn is NULL");
  if (n_layers < 1) return fail(MOE_EINVAL, "n_layers = %d", n_layers);
  int st;
  for (int l = 0; l < n_layers; ++l) {
    if ((st = check_layer(&layers[l])) != MOE_OK) return st;
    const moe_layer_t &a = layers[0], &b = layers[l];
    if (a.hidden != b.hidden || a.inter != b.inter || a.n_experts != b.n_experts ||
        a.top_k != b.top_k || a.bits_routed != b.bits_routed || a.bits_shared != b.bits_shared ||
        a.router_dtype != b.router_dtype || a.gate_dtype != b.gate_dtype)
      return fail(MOE_EINVAL, "layer %d differs in shape or format from layer 0", l);
    if (gdn[l].state && (st = check_gdn(&layers[l], &gdn[l], l)) != MOE_OK) return st;
  }
  if ((st = check_vec(h, "h")) != MOE_OK) return st;
  if (updates_bf16 && !aligned(updates_bf16, 16)) return fail(MOE_EALIGN, "updates must be 16-byte aligned");
  if (!idx_log || !w_log) return fail(MOE_EINVAL, "idx_log / w_log is NULL");
  if (!aligned(idx_log, 4) || !aligned(w_log, 4)) return fail(MOE_EALIGN, "logs must be 4-byte aligned");
  const moe_layer_t *L = &layers[0];
  int D, heads;
  gdn_extent(gdn, n_layers, D, heads);
  const WsLayout wl = ws_layout(L, 1, n_layers, D, heads);
  if ((st = check_ws(ws, ws_bytes, wl.total)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t *wsb = static_cast<uint8_t *>(ws);
  float *pong = reinterpret_cast<float *>(wsb + wl.h_pong);
  float *hg = reinterpret_cast<float *>(wsb + wl.gdn_h);
  const size_t H = L->hidden, K = L->top_k;
  float *cur = h, *nxt = pong;
  for (int l = 0; l < n_layers; ++l) {
    const float *h_in = cur;
    const uint16_t *u = nullptr;
    if (gdn[l].state) {
      if ((st = gdn_block(&layers[l], &gdn[l], cur, hg, wsb, wl, s)) != MOE_OK) return st;
      h_in = hg;
    } else if (updates_bf16) {
      u = updates_bf16 + (size_t)l * H;
    }
    st = layer_token(&layers[l], XS_NORM, nullptr, h_in, u, nullptr, nxt, idx_log + l * K,
                     w_log + l * K, wsb, wl, s);
    if (st != MOE_OK) return st;
    float *t = cur;
    cur = nxt;
    nxt = t;
  }
  if (cur != h)
    MOE_TRY_HIP(timed(s, MOE_KERNEL_OTHER, [&] { return launch_copy_f32(h, cur, L->hidden, s); }), "copy launch");
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// host-memory expert tier: the routed records in page-locked host memory, a
// cache of n_slots records and the slot table in device memory, all managed
// on the device (no host round trip, so a token's calls can be captured)
// ---------------------------------------------------------------------------
struct moe_tier_s {
  const uint8_t *host;       // as given
  const uint8_t *host_dev;   // its device address
  int E;
  size_t stride;
  uint8_t *cache;
  int n_slots;
  uint8_t *state;
};

size_t moe_tier_state_bytes(int n_experts, int n_slots) {
  if (n_experts < 1 || n_experts > kMaxE || n_slots < kMaxK || n_slots > n_experts) return 0;
  return up256(kTierOwnerOff + (size_t)n_slots * 8);
}

int moe_tier_create(const void *host_records, int n_experts, size_t expert_stride, void *cache,
                    int n_slots, void *state, moe_tier_t *out) {
  if (!out) return fail(MOE_EINVAL, "out is NULL");
  if (!host_records || !cache || !state) return fail(MOE_EINVAL, "host_records / cache / state is NULL");
  if (n_experts < 1 || n_experts > kMaxE) return fail(MOE_EINVAL, "n_experts = %d: need 1..1024", n_experts);
  if (n_slots < kMaxK || n_slots > n_experts)
    return fail(MOE_EINVAL, "n_slots = %d: need 8..n_experts", n_slots);
  if (expert_stride == 0 || expert_stride % 256 || !aligned(cache, 256) || !aligned(state, 256) ||
      !aligned(host_records, 256))
    return fail(MOE_EALIGN, "host_records, cache, state and expert_stride must be 256-byte aligned");
  // the kernels read missing records from host memory through its device
  // address: only page-locked memory the device can map has one
  void *dev = nullptr;
  const hipError_t e = hipHostGetDevicePointer(&dev, const_cast<void *>(host_records), 0);
  if (e != hipSuccess || !dev)
    return fail(MOE_EINVAL, "host_records must be page-locked host memory the device can read "
                "(hipHostMalloc): %s", hipGetErrorString(e));
  moe_tier_s *t = new moe_tier_s;
  t->host = static_cast<const uint8_t *>(host_records);
  t->host_dev = static_cast<const uint8_t *>(dev);
  t->E = n_experts;
  t->stride = expert_stride;
  t->cache = static_cast<uint8_t *>(cache);
  t->n_slots = n_slots;
  t->state = static_cast<uint8_t *>(state);
  *out = t;
  return MOE_OK;
}

int moe_tier_destroy(moe_tier_t t) {
  if (!t) return fail(MOE_EINVAL, "tier is NULL");
  delete t;
  return MOE_OK;
}

int moe_tier_reset(moe_tier_t t, void *stream) {
  if (!t) return fail(MOE_EINVAL, "tier is NULL");
  MOE_TRY_HIP(debug_check(static_cast<hipStream_t>(stream),
                          launch_tier_reset(t->state, t->n_slots, static_cast<hipStream_t>(stream))),
              "tier reset launch");
  return MOE_OK;
}

int moe_tier_stats(moe_tier_t t, void *stream, unsigned long long *hits, unsigned long long *misses,
                   unsigned long long *bytes_read, int32_t *slot_owner) {
  if (!t) return fail(MOE_EINVAL, "tier is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  TierState st;
  MOE_TRY_HIP(hipMemcpyAsync(&st, t->state, sizeof st, hipMemcpyDeviceToHost, s), "tier state copy");
  if (slot_owner)
    MOE_TRY_HIP(hipMemcpyAsync(slot_owner, t->state + kTierOwnerOff, sizeof(int32_t) * t->n_slots,
                               hipMemcpyDeviceToHost, s), "tier slot copy");
  MOE_TRY_HIP(hipStreamSynchronize(s), "waiting for the tier state");
  if (hits) *hits = st.hits;
  if (misses) *misses = st.misses;
  if (bytes_read) *bytes_read = st.bytes;
  return MOE_OK;
}

int moe_tier_layer_decode(const moe_layer_t *L, moe_tier_t t, moe_dtype x_dtype, const void *x,
                          const float *h_res, float *h_out, int32_t *topk_idx, float *topk_w,
                          void *ws, size_t ws_bytes, void *stream) {
  if (!L) return fail(MOE_EINVAL, "layer is NULL");
  if (!t) return fail(MOE_EINVAL, "tier is NULL");
  moe_layer_t Lc = *L;  // the routed records come from the tier
  Lc.experts = t->cache;
  Lc.expert_stride = t->stride;
  int st;
  if ((st = check_layer(&Lc)) != MOE_OK) return st;
  if (t->E != L->n_experts)
    return fail(MOE_EINVAL, "the tier holds %d experts, the layer has %d", t->E, L->n_experts);
  const size_t rb = moe_expert_bytes(L->hidden, L->inter, L->bits_routed, L->group);
  if (t->stride < rb) return fail(MOE_EINVAL, "tier stride %zu < record size %zu", t->stride, rb);
  if (L->top_k > t->n_slots) return fail(MOE_EINVAL, "top_k %d > tier slots %d", L->top_k, t->n_slots);
  if ((st = check_dtype(x_dtype, "x_dtype")) != MOE_OK) return st;
  if ((st = check_vec(x, "x")) != MOE_OK) return st;
  if ((st = check_vec(h_res, "h_res")) != MOE_OK) return st;
  if ((st = check_vec(h_out, "h_out")) != MOE_OK) return st;
  if (h_out == h_res) return fail(MOE_EINVAL, "h_out may not alias h_res");
  if (!topk_idx || !topk_w) return fail(MOE_EINVAL, "topk_idx / topk_w is NULL");
  if (!aligned(topk_idx, 4) || !aligned(topk_w, 4)) return fail(MOE_EALIGN, "topk outputs must be 4-byte aligned");
  const WsLayout wl = ws_layout(L, 1, 0);
  if ((st = check_ws(ws, ws_bytes, wl.total)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t *wsb = static_cast<uint8_t *>(ws);
  float *logits = reinterpret_cast<float *>(wsb + wl.logits);
  float *sigma = reinterpret_cast<float *>(wsb + wl.sigma);
  float *h_routed = reinterpret_cast<float *>(wsb + wl.h_routed);
  float *h_shared = reinterpret_cast<float *>(wsb + wl.h_shared);
  float *y_shared = reinterpret_cast<float *>(wsb + wl.y_shared);
  int32_t *slot_ids = reinterpret_cast<int32_t *>(wsb + wl.ids);
  uint64_t *rec_src = reinterpret_cast<uint64_t *>(wsb + wl.rec_src);
  uint64_t *rec_fill = rec_src + kMaxK;
  const int K = L->top_k;
  const int xsrc = x_dtype == MOE_BF16 ? XS_BF16 : XS_F32;
  const bool same = L->bits_shared == L->bits_routed;

  // router rows, shared gate (and the shared gate/up at another width)
  HeadParams hp = head_params(&Lc, 1);
  hp.xsrc = xsrc;
  hp.x = x;
  hp.logits = logits;
  hp.sigma = sigma;
  hp.h_shared = h_shared;
  hp.n_shared_waves = same ? 0 : 1;
  hp.bits_routed = L->bits_routed;
  MOE_TRY_HIP(timed(s, MOE_KERNEL_HEAD, [&] { return launch_head(hp, s); }), "router launch");
  // top-K and the slot of every selected expert, on the device
  TierRouteParams tp;
  tp.logits = logits;
  tp.E = L->n_experts;
  tp.K = K;
  tp.renorm = L->renorm_topk;
  tp.n_slots = t->n_slots;
  tp.state = t->state;
  tp.host_dev = t->host_dev;
  tp.cache = t->cache;
  tp.stride = t->stride;
  tp.record_bytes = rb;
  tp.idx = topk_idx;
  tp.w = topk_w;
  tp.slot = slot_ids;
  tp.rec_src = rec_src;
  tp.rec_fill = rec_fill;
  MOE_TRY_HIP(timed(s, MOE_KERNEL_TOPK, [&] { return launch_tier_route(tp, s); }), "tier routing launch");

  // gate/up of the slots' records (hits from the cache, misses from host
  // memory, written into their slots) + the shared expert, down + combine
  GateUpParams gp;
  memset(&gp, 0, sizeof gp);
  gp.H = L->hidden;
  gp.I = L->inter;
  gp.E = t->n_slots;
  gp.K = K;
  gp.bits = L->bits_routed;
  gp.experts = t->cache;
  gp.stride = t->stride;
  gp.shared_rec = static_cast<const uint8_t *>(L->shared_expert);
  gp.shared_ok = same;
  gp.off = offsets_of(L->hidden, L->inter, L->bits_routed);
  gp.soff = offsets_of(L->hidden, L->inter, L->bits_shared);
  gp.ids = slot_ids;
  gp.n = K;
  gp.xsrc = xsrc;
  gp.x = x;
  gp.h_out = h_routed;
  gp.with_shared = same;
  gp.h_shared_out = h_shared;
  gp.rec_src = rec_src;
  gp.rec_fill = rec_fill;
  MOE_TRY_HIP(timed(s, MOE_KERNEL_GATEUP, [&] { return launch_gateup(gp, s); }), "gate/up launch");
  DownParams dp;
  memset(&dp, 0, sizeof dp);
  dp.H = L->hidden;
  dp.I = L->inter;
  dp.E = t->n_slots;
  dp.experts = t->cache;
  dp.stride = t->stride;
  dp.shared_rec = gp.shared_rec;
  dp.off = gp.off;
  dp.soff = gp.soff;
  dp.shared_ok = 1;
  if (!same) {
    DownParams sp = dp;
    sp.combine = 0;
    sp.bits_r = L->bits_shared;
    sp.ids = nullptr;
    sp.n = 1;
    sp.h = h_shared;
    sp.y = y_shared;
    MOE_TRY_HIP(timed(s, MOE_KERNEL_DOWN_Y, [&] { return launch_down(sp, s); }), "shared down launch");
  }
  dp.combine = 1;
  dp.bits_r = L->bits_routed;
  dp.bits_s = L->bits_shared;
  dp.idx = slot_ids;
  dp.w = topk_w;
  dp.K = K;
  dp.sigma = sigma;
  dp.h_routed = h_routed;
  dp.h_shared = same ? h_shared : nullptr;
  dp.y = same ? nullptr : y_shared;
  dp.h_res = h_res;
  dp.out = h_out;
  // the gate/up launch has filled every missing record's slot, down rows
  // included: the down kernel reads all routed records from their slots
  MOE_TRY_HIP(timed(s, MOE_KERNEL_DOWN, [&] { return launch_down(dp, s); }), "down/combine launch");
  return MOE_OK;
}

struct moe_graph_s {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

int moe_graph_capture_begin(void *stream) {
  if (!stream) return fail(MOE_EINVAL, "capture needs a non-NULL stream");
  MOE_TRY_HIP(hipStreamBeginCapture(static_cast<hipStream_t>(stream), hipStreamCaptureModeThreadLocal),
              "hipStreamBeginCapture");
  return MOE_OK;
}

int moe_graph_capture_end(void *stream, moe_graph_t *out) {
  if (!stream || !out) return fail(MOE_EINVAL, "stream / out is NULL");
  hipGraph_t g = nullptr;
  MOE_TRY_HIP(hipStreamEndCapture(static_cast<hipStream_t>(stream), &g), "hipStreamEndCapture");
  hipGraphExec_t ex = nullptr;
  hipError_t e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(g);
    return hip_fail(e, "hipGraphInstantiate");
  }
  moe_graph_s *r = new moe_graph_s{g, ex};
  *out = r;
  return MOE_OK;
}

int moe_graph_create_stack(const moe_layer_t *layers, int n_layers, const uint16_t *updates_bf16,
                           float *h, int32_t *idx_log, float *w_log, void *ws, size_t ws_bytes,
                           void *stream, moe_graph_t *out) {
  if (!out) return fail(MOE_EINVAL, "out is NULL");
  int st = moe_graph_capture_begin(stream);
  if (st != MOE_OK) return st;
  st = moe_stack_decode(layers, n_layers, updates_bf16, h, idx_log, w_log, ws, ws_bytes, stream);
  if (st != MOE_OK) {
    hipGraph_t g = nullptr;
    (void)hipStreamEndCapture(static_cast<hipStream_t>(stream), &g);
    if (g) (void)hipGraphDestroy(g);
    return st;
  }
  return moe_graph_capture_end(stream, out);
}

int moe_graph_launch(moe_graph_t g, void *stream) {
  if (!g) return fail(MOE_EINVAL, "graph is NULL");
  MOE_TRY_HIP(hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream)), "hipGraphLaunch");
  return MOE_OK;
}

int moe_graph_destroy(moe_graph_t g) {
  if (!g) return fail(MOE_EINVAL, "graph is NULL");
  (void)hipGraphExecDestroy(g->exec);
  (void)hipGraphDestroy(g->graph);
  delete g;
  return MOE_OK;
}

int moe_gdn_step(int n_seq, int n_heads, int d_k, int d_v, const float *q, const float *k,
                 const float *v, const float *alpha, const float *beta, float *state,
                 float *out, void *stream) {
  if (n_seq < 1 || n_heads < 1) return fail(MOE_EINVAL, "n_seq = %d, n_heads = %d: need >= 1", n_seq, n_heads);
  if ((long long)n_seq * n_heads > (1 << 24)) return fail(MOE_EINVAL, "n_seq * n_heads too large");
  if (d_k != 16 && d_k != 32 && d_k != 64 && d_k != 128 && d_k != 256)
    return fail(MOE_EUNSUPPORTED, "d_k = %d: only 16, 32, 64, 128 and 256 are built", d_k);
  if (d_v < 1 || d_v > kMaxDim) return fail(MOE_EINVAL, "d_v = %d: need 1..%d", d_v, kMaxDim);
  if (!q || !k || !v || !alpha || !beta || !state || !out) return fail(MOE_EINVAL, "a pointer is NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(state, 16))
    return fail(MOE_EALIGN, "q, k and state must be 16-byte aligned");
  if (!aligned(v, 4) || !aligned(alpha, 4) || !aligned(beta, 4) || !aligned(out, 4))
    return fail(MOE_EALIGN, "v, alpha, beta and out must be 4-byte aligned");
  GdnParams p;
  p.n_sh = n_seq * n_heads;
  p.d_k = d_k;
  p.d_v = d_v;
  p.q = q;
  p.k = k;
  p.v = v;
  p.alpha = alpha;
  p.beta = beta;
  p.state = state;
  p.out = out;
  p.prep = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  MOE_TRY_HIP(timed(s, MOE_KERNEL_GDN_STEP, [&] { return launch_gdn_step(p, s); }), "delta-rule step launch");
  return MOE_OK;
}

int moe_fill_experts(void *dst, size_t stride, int n, uint64_t seed, int layer, int first_expert,
                     int hidden, int inter, int bits, double scale_lo, double scale_hi,
                     double bias_lo, double bias_hi, void *stream) {
  if (!dst) return fail(MOE_EINVAL, "dst is NULL");
  if (!aligned(dst, 256) || stride % 256) return fail(MOE_EALIGN, "dst and stride must be 256-byte aligned");
  int st;
  if ((st = check_bits(bits, "bits")) != MOE_OK) return st;
  if (!dim_ok(hidden) || !dim_ok(inter)) return fail(MOE_EINVAL, "hidden/inter must be multiples of 64 in [64, 8192]");
  if (n < 1 || n > 65535) return fail(MOE_EINVAL, "n = %d: need 1..65535", n);
  const RecOffsets off = record_offsets(hidden, inter, bits);
  if (n > 1 && stride < off.total) return fail(MOE_EINVAL, "stride %zu < record size %zu", stride, off.total);
  if (!(scale_lo <= scale_hi) || !(bias_lo <= bias_hi)) return fail(MOE_EINVAL, "empty value range");
  FillParams p;
  p.dst = static_cast<uint8_t *>(dst);
  p.stride = stride;
  p.n = n;
  p.seed = seed;
  p.layer = layer;
  p.first_expert = first_expert;
  p.H = hidden;
  p.I = inter;
  p.bits = bits;
  p.scale_lo = scale_lo;
  p.scale_hi = scale_hi;
  p.bias_lo = bias_lo;
  p.bias_hi = bias_hi;
  p.off = off;
  MOE_TRY_HIP(debug_check(static_cast<hipStream_t>(stream), launch_fill(p, static_cast<hipStream_t>(stream))),
              "fill launch");
  return MOE_OK;
}

int moe_profile_begin(int max_launches) {
  if (max_launches < 1 || max_launches > (1 << 20)) return fail(MOE_EINVAL, "max_launches = %d", max_launches);
  if (g_prof.on) return fail(MOE_EINVAL, "profiling already active on this thread");
  g_prof.ev.assign(2 * (size_t)max_launches, nullptr);
  g_prof.ids.assign(max_launches, 0);
  for (auto &e : g_prof.ev) {
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      for (auto &f : g_prof.ev)
        if (f) (void)hipEventDestroy(f);
      g_prof.ev.clear();
      return hip_fail(r, "hipEventCreate");
    }
  }
  g_prof.cap = max_launches;
  g_prof.n = 0;
  g_prof.on = true;
  return MOE_OK;
}

int moe_profile_end(float *ms, int *kernel_ids, int capacity, int *n_out) {
  if (!g_prof.on) return fail(MOE_EINVAL, "profiling is not active on this thread");
  if (!n_out || (capacity > 0 && !ms)) return fail(MOE_EINVAL, "output pointer is NULL");
  int st = MOE_OK;
  const int n = g_prof.n < capacity ? g_prof.n : capacity;
  if (g_prof.n > 0) {
    hipError_t r = hipEventSynchronize(g_prof.ev[2 * (g_prof.n - 1) + 1]);
    if (r != hipSuccess) st = hip_fail(r, "hipEventSynchronize");
  }
  for (int i = 0; i < n && st == MOE_OK; ++i) {
    float t = 0.f;
    hipError_t r = hipEventElapsedTime(&t, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]);
    if (r != hipSuccess) st = hip_fail(r, "hipEventElapsedTime");
    ms[i] = t;
    if (kernel_ids) kernel_ids[i] = g_prof.ids[i];
  }
  *n_out = st == MOE_OK ? n : 0;
  for (auto &e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.clear();
  g_prof.ids.clear();
  g_prof.on = false;
  g_prof.n = g_prof.cap = 0;
  return st;
}

int moe_zero(void *ptr, size_t bytes, void *stream) {
  if (!ptr) return fail(MOE_EINVAL, "ptr is NULL");
  if (!aligned(ptr, 16)) return fail(MOE_EALIGN, "ptr must be 16-byte aligned");
  MOE_TRY_HIP(debug_check(static_cast<hipStream_t>(stream), launch_zero(ptr, bytes, static_cast<hipStream_t>(stream))),
              "zero launch");
  return MOE_OK;
}

}  // extern "C"
