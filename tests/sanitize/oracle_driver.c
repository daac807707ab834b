/* Host sanitizer driver for the fp64 oracle (test infrastructure): runs the
 * layer, the decode step and the linear-attention block on small synthetic
 * inputs, built with AddressSanitizer and UndefinedBehaviorSanitizer, so that
 * an out-of-bounds access, a use after free or undefined arithmetic in the
 * oracle stops the run. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

size_t oracle_record_bytes(int hidden, int inter, int bits);
void oracle_layer(int hidden, int inter, int n_experts, int top_k, int bits_routed,
                  int bits_shared, int renorm, int router_dtype, const void *router,
                  int gate_dtype, const void *gate_vec, const uint8_t *experts,
                  size_t expert_stride, const uint8_t *shared_record, const double *x,
                  const double *h_res, double *logits, double *p, int32_t *idx, double *w,
                  double *sigma, double *h, double *y, double *out);
void oracle_gdn_step(int n_seq, int n_heads, int d_k, int d_v, const double *q,
                     const double *k, const double *v, const double *alpha,
                     const double *beta, double *state, double *out);
void oracle_gdn_block(int hidden, int n_heads, int d_head, int bits, const uint8_t *rec_qko,
                      const uint8_t *rec_vab, const double *h, double *state, double *proj,
                      double *o, double *h_out);
void oracle_set_threads(int n);

static uint64_t g_state = 0x243F6A8885A308D3ull;
static uint32_t next_u32(void) {  /* 64-bit LCG (Knuth's MMIX constants), high half */
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(g_state >> 32);
}
static double uniform(double lo, double hi) { return lo + (hi - lo) * (next_u32() / 4294967296.0); }
static uint16_t bf16_of(double v) {  /* truncation is enough for test data */
  float f = (float)v;
  uint32_t b;
  memcpy(&b, &f, 4);
  return (uint16_t)(b >> 16);
}

/* a record of `bytes` bytes: random code words, sb words of small bf16 pairs */
static uint8_t *record(size_t bytes, size_t n_records) {
  uint8_t *r = (uint8_t *)malloc(bytes * n_records);
  uint32_t *w = (uint32_t *)r;
  for (size_t i = 0; i < bytes * n_records / 4; ++i)
    w[i] = (uint32_t)bf16_of(uniform(0.001, 0.01)) | ((uint32_t)bf16_of(uniform(-0.02, 0.02)) << 16);
  return r;
}

static double checksum = 0.0;

static void run_layer(int H, int I, int E, int K, int bits, int router_dtype) {
  const size_t rb = oracle_record_bytes(H, I, bits);
  uint8_t *experts = record(rb, (size_t)E), *shared = record(rb, 1);
  void *router;
  if (router_dtype == 1) {
    uint16_t *r = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)E * H);
    for (size_t i = 0; i < (size_t)E * H; ++i) r[i] = bf16_of(uniform(-0.05, 0.05));
    router = r;
  } else {
    float *r = (float *)malloc(sizeof(float) * (size_t)E * H);
    for (size_t i = 0; i < (size_t)E * H; ++i) r[i] = (float)uniform(-0.05, 0.05);
    router = r;
  }
  float *gate = (float *)malloc(sizeof(float) * H);
  double *x = (double *)malloc(sizeof(double) * H), *hres = (double *)malloc(sizeof(double) * H);
  for (int i = 0; i < H; ++i) {
    gate[i] = (float)uniform(-0.05, 0.05);
    x[i] = uniform(-1.0, 1.0);
    hres[i] = uniform(-1.0, 1.0);
  }
  double *logits = (double *)malloc(sizeof(double) * E), *p = (double *)malloc(sizeof(double) * E);
  int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * K);
  double *w = (double *)malloc(sizeof(double) * K), sigma = 0.0;
  double *h = (double *)malloc(sizeof(double) * (size_t)(K + 1) * I);
  double *y = (double *)malloc(sizeof(double) * (size_t)(K + 1) * H);
  double *out = (double *)malloc(sizeof(double) * H);
  oracle_layer(H, I, E, K, bits, bits, 1, router_dtype, router, 0, gate, experts, rb, shared, x, hres,
               logits, p, idx, w, &sigma, h, y, out);
  for (int i = 0; i < H; ++i) checksum += out[i];
  free(experts); free(shared); free(router); free(gate); free(x); free(hres); free(logits); free(p);
  free(idx); free(w); free(h); free(y); free(out);
}

static void run_gdn(int H, int heads, int d, int bits) {
  const int D = heads * d;
  const size_t rb = oracle_record_bytes(H, D, bits);
  uint8_t *qko = record(rb, 1), *vab = record(rb, 1);
  double *hv = (double *)malloc(sizeof(double) * H), *hout = (double *)malloc(sizeof(double) * H);
  double *state = (double *)malloc(sizeof(double) * (size_t)heads * d * d);
  double *proj = (double *)malloc(sizeof(double) * (size_t)(3 * D + 2 * heads));
  double *o = (double *)malloc(sizeof(double) * D);
  for (int i = 0; i < H; ++i) hv[i] = uniform(-1.0, 1.0);
  for (size_t i = 0; i < (size_t)heads * d * d; ++i) state[i] = uniform(-0.01, 0.01);
  oracle_gdn_block(H, heads, d, bits, qko, vab, hv, state, proj, o, hout);
  for (int i = 0; i < H; ++i) checksum += hout[i];
  /* the step alone, two sequences */
  const int S = 2;
  double *q = (double *)malloc(sizeof(double) * S * D), *k = (double *)malloc(sizeof(double) * S * D);
  double *v = (double *)malloc(sizeof(double) * S * D), *al = (double *)malloc(sizeof(double) * S * heads);
  double *be = (double *)malloc(sizeof(double) * S * heads);
  double *st = (double *)malloc(sizeof(double) * (size_t)S * heads * d * d);
  double *so = (double *)malloc(sizeof(double) * S * D);
  for (int i = 0; i < S * D; ++i) { q[i] = uniform(-1, 1); k[i] = uniform(-1, 1); v[i] = uniform(-1, 1); }
  for (int i = 0; i < S * heads; ++i) { al[i] = uniform(0.5, 1.0); be[i] = uniform(0.0, 1.0); }
  for (size_t i = 0; i < (size_t)S * heads * d * d; ++i) st[i] = uniform(-0.01, 0.01);
  oracle_gdn_step(S, heads, d, d, q, k, v, al, be, st, so);
  for (int i = 0; i < S * D; ++i) checksum += so[i];
  free(qko); free(vab); free(hv); free(hout); free(state); free(proj); free(o);
  free(q); free(k); free(v); free(al); free(be); free(st); free(so);
}

int main(void) {
  oracle_set_threads(2);
  run_layer(128, 64, 8, 2, 4, 1);
  run_layer(128, 64, 8, 2, 2, 0);
  run_layer(192, 320, 16, 4, 4, 1);  /* rows that do not fill 64 lanes */
  run_gdn(128, 2, 32, 4);
  run_gdn(128, 2, 32, 2);
  if (!isfinite(checksum)) {
    printf("oracle checksum not finite\n");
    return 1;
  }
  printf("oracle ok %.6e\n", checksum);
  return 0;
}
