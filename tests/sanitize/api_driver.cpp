// Host sanitizer driver for the validation layer (test infrastructure): calls
// every entry point with arguments its checks must refuse, and with valid
// arguments that end at a (stubbed) launch, built with AddressSanitizer and
// UndefinedBehaviorSanitizer.  No device is touched: pointers are never
// dereferenced by the host code, streams are NULL.
#include <stdio.h>
#include <string.h>

#include "../../include/moe.h"

static int n_checks = 0, n_bad = 0;
static void expect(int got, int want, const char *what) {
  ++n_checks;
  if (got != want) {
    ++n_bad;
    printf("%s: got %d want %d (%s)\n", what, got, want, moe_last_error());
  }
}
static void expect_fail(int got, const char *what) {
  ++n_checks;
  if (got >= 0) {
    ++n_bad;
    printf("%s: accepted (%d)\n", what, got);
  }
  if (strlen(moe_last_error()) == 0) {
    ++n_bad;
    printf("%s: no message\n", what);
  }
}

static moe_layer_t layer(void) {
  moe_layer_t L;
  memset(&L, 0, sizeof L);
  L.hidden = 4096; L.inter = 1024; L.n_experts = 512; L.top_k = 4; L.group = 64;
  L.bits_routed = 4; L.bits_shared = 4; L.renorm_topk = 1;
  L.router_dtype = MOE_BF16; L.router = (const void *)0x100000;
  L.gate_dtype = MOE_BF16; L.shared_gate = (const void *)0x200000;
  L.experts = (const void *)0x10000000; L.expert_stride = moe_expert_bytes(4096, 1024, 4, 64);
  L.shared_expert = (const void *)0x300000;
  return L;
}

int main(void) {
  for (int s = -6; s <= 1; ++s) (void)strlen(moe_strerror(s));
  (void)moe_abi_version();
  size_t off[6];
  expect(moe_expert_offsets(4096, 1024, 4, 64, off), MOE_OK, "offsets");
  expect_fail(moe_expert_offsets(4096, 1024, 3, 64, off), "offsets bits 3");
  expect(moe_expert_bytes(100, 1024, 4, 64) == 0, 1, "record of a bad shape");
  expect(moe_qmatrix_bytes(1024, 4096, 2, 64) > 0, 1, "matrix bytes");

  moe_layer_t L = layer();
  const size_t ws_need = moe_layer_workspace_bytes(&L, 1);
  expect(ws_need > 0, 1, "workspace bytes");
  void *ws = (void *)0x40000000;
  const void *x = (const void *)0x500000;
  float *hres = (float *)0x600000, *hout = (float *)0x700000, *w = (float *)0x900000;
  int32_t *idx = (int32_t *)0x800000;
  // refused arguments
  expect_fail(moe_layer_decode(NULL, 1, MOE_BF16, x, hres, hout, idx, w, ws, ws_need, NULL), "null layer");
  moe_layer_t B = L; B.group = 32;
  expect_fail(moe_layer_decode(&B, 1, MOE_BF16, x, hres, hout, idx, w, ws, ws_need, NULL), "group 32");
  B = L; B.router_tiles = (const void *)0x100008;
  expect_fail(moe_layer_decode(&B, 1, MOE_BF16, x, hres, hout, idx, w, ws, ws_need, NULL), "tiles misaligned");
  expect_fail(moe_layer_decode(&L, 0, MOE_BF16, x, hres, hout, idx, w, ws, ws_need, NULL), "no tokens");
  expect_fail(moe_layer_decode(&L, 1, MOE_BF16, x, hres, hout, idx, w, ws, ws_need - 1, NULL), "small ws");
  expect_fail(moe_layer_decode(&L, 1, MOE_BF16, x, hres, hres, idx, w, ws, ws_need, NULL), "aliasing");
  // accepted: ends at the stubbed launch
  expect(moe_layer_decode(&L, 1, MOE_BF16, x, hres, hout, idx, w, ws, ws_need, NULL), MOE_EHIP, "launch");
  expect(moe_layer_decode_noalloc(&L, 1, MOE_BF16, x, hres, hout, idx, w, NULL), MOE_EHIP, "noalloc");
  expect_fail(moe_route(&L, 65, MOE_BF16, x, idx, w, w, NULL, ws, ws_need, NULL), "route 65 tokens");
  expect_fail(moe_expert_forward_q4(&L, MOE_BF16, x, idx, 0, hout, NULL, ws, ws_need, NULL), "no experts");
  expect_fail(moe_expert_forward_q2(&L, MOE_BF16, x, idx, 2, hout, NULL, ws, ws_need, NULL), "q2 entry, q4 layer");
  expect_fail(moe_combine(4096, 9, hres, hout, w, hout, w, hres, NULL), "combine K 9");
  moe_ws_view v;
  expect(moe_layer_ws_view(&L, 1, ws, ws_need, &v), MOE_OK, "ws view");

  // stacks
  moe_layer_t S[3] = {L, L, L};
  const size_t sws = moe_stack_workspace_bytes(S, 3);
  expect(sws > 0, 1, "stack workspace");
  float *h = (float *)0x700000;
  expect(moe_stack_decode(S, 3, NULL, h, idx, w, ws, sws, NULL), MOE_EHIP, "stack launch");
  S[1].inter = 512;
  expect_fail(moe_stack_decode(S, 3, NULL, h, idx, w, ws, sws, NULL), "mixed stack");
  moe_gdn_layer_t G[3];
  memset(G, 0, sizeof G);
  G[0].n_heads = 64; G[0].d_head = 128; G[0].bits = 4;
  G[0].rec_qko = (const void *)0x20000000; G[0].rec_vab = (const void *)0x30000000;
  G[0].state = (float *)0x38000000;
  S[1] = L;
  const size_t gws = moe_stack_gdn_workspace_bytes(S, G, 3);
  expect(gws > 0, 1, "gdn stack workspace");
  expect(moe_stack_decode_gdn(S, G, 3, NULL, h, idx, w, ws, gws, NULL), MOE_EHIP, "gdn stack launch");
  G[0].d_head = 100;
  expect_fail(moe_stack_decode_gdn(S, G, 3, NULL, h, idx, w, ws, gws, NULL), "gdn head width");
  expect_fail(moe_router_tile(NULL, 512, 4096, MOE_BF16, (void *)0x700000, NULL), "tile null");
  expect(moe_router_tile((const void *)0x100000, 512, 4096, MOE_BF16, (void *)0x10000000, NULL), MOE_EHIP,
         "tile launch");

  // tier: a host pointer the device cannot map is refused
  static char host[8192];
  moe_tier_t t = NULL;
  expect(moe_tier_state_bytes(512, 128) > 0, 1, "tier state bytes");
  expect_fail(moe_tier_create(host, 16, 256, (void *)0x100000, 8, (void *)0x200000, &t), "tier host memory");
  expect_fail(moe_tier_create(NULL, 16, 256, (void *)0x100000, 8, (void *)0x200000, &t), "tier null");
  expect_fail(moe_tier_destroy(NULL), "tier destroy null");

  // decode step, fill, zero, graphs
  const float *f = (const float *)0x100000;
  expect_fail(moe_gdn_step(1, 0, 128, 128, f, f, f, f, f, (float *)0x200000, (float *)0x300000, NULL), "no heads");
  expect(moe_gdn_step(1, 2, 128, 128, f, f, f, f, f, (float *)0x200000, (float *)0x300000, NULL), MOE_EHIP,
         "gdn launch");
  expect_fail(moe_fill_experts(NULL, 256, 1, 1, 0, 0, 4096, 1024, 4, 0.1, 0.2, 0.0, 0.1, NULL), "fill null");
  expect_fail(moe_zero(NULL, 16, NULL), "zero null");
  expect_fail(moe_graph_capture_begin(NULL), "capture on the NULL stream");
  expect_fail(moe_graph_launch(NULL, NULL), "launch a null graph");
  int n_out = 0;
  expect_fail(moe_profile_end(NULL, NULL, 0, &n_out), "profile end without begin");

  printf("api %s: %d checks, %d failed\n", n_bad ? "FAILED" : "ok", n_checks, n_bad);
  return n_bad ? 1 : 0;
}
