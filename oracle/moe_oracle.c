/*
 * moe_oracle.c -- plain, slow, fp64 CPU reference of the MoE expert forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this.  It shares no code, header,
 * table or constant with the HIP library: the record format is decoded here
 * from its definition, independently.
 *
 * Every quantity is the plain definition evaluated in fp64 with one fixed,
 * sequential summation order (compiled with -ffp-contract=off, no fast math).
 * bf16 -> fp64 and code -> fp64 conversions are exact.  OpenMP, when enabled,
 * only splits independent output rows, so results are bitwise equal to a
 * serial run.
 *
 * Pages (cited by site and section):
 *   [openclawradar] openclawradar.com (ja), "Flash-MoE: running the 397B
 *       parameter Qwen model on a MacBook Pro in pure C/Metal"
 *   [a2a-fr] a2a-mcp.org (fr), "What is Flash-MoE? Running 397B-parameter AI
 *       models on a laptop"
 *   [sardonic] education.sardonicrepulsion.com (sk), "Flash-MoE: how to run a
 *       397-billion-parameter AI model on an ordinary notebook"
 *
 * Readings taken where the pages are silent:
 *   - codes are unsigned, little-endian inside 32-bit words: element c of a row
 *     sits in word c*b/32 at bit b*(c mod 32/b); rows are contiguous;
 *   - one (scale, bias) pair per 64 consecutive input columns, stored as a
 *     32-bit word with the bf16 scale in the low half and the bf16 bias in the
 *     high half;
 *   - selection is on the logits (softmax is monotone), exact ties go to the
 *     lower expert index, output order is descending probability;
 *   - renormalising the K selected probabilities is a flag;
 *   - the shared expert is gated by the scalar sigmoid(g . x);
 *   - SwiGLU applies silu to the gate projection: h = silu(gate x) * (up x);
 *   - RMSNorm has unit weight and eps 1e-6;
 *   - the linear-attention decode step is the gated delta rule in the order
 *     of the pages' BLAS calls: scale the state, u = S k, S += beta (v - u) k^T,
 *     o = S q, with q, k, v, alpha, beta given (their projections are not part
 *     of this step);
 *   - a linear-attention block around it (the pages give only the head count
 *     and state size): x = RMSNorm(h); q, k, v and one alpha and one beta
 *     logit per head are rows of quantised projections of x; q and k are
 *     scaled to unit length per head (eps 1e-6 under the root), alpha and
 *     beta are sigmoids of their logits; the block adds the quantised output
 *     projection of o to the residual stream.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_GROUP 64

/* Threads of the row loops (timing only: each output row is summed by one
 * thread in its fixed order, so the results do not depend on it). */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* scalar helpers                                                      */
/* ------------------------------------------------------------------ */
static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* code of column c of a packed row (b-bit unsigned, see header) */
static unsigned code_of(const uint32_t *row_words, int c, int bits)
{
    int per_word = 32 / bits;
    uint32_t w = row_words[c / per_word];
    return (w >> (bits * (c % per_word))) & ((1u << bits) - 1u);
}

/* Dequantised weight: w = q * scale + bias, with (scale, bias) of the group
 * that holds column c.  [a2a-fr] "FMA-optimised dequantisation kernels" and
 * [openclawradar] "FMA-optimized dequant kernel" give this naive form; the
 * FMA rewrites they describe are regroupings of the same product. */
static double dequant(const uint32_t *codes, const uint32_t *sb, int cols,
                      int bits, int r, int c)
{
    const uint32_t *row = codes + (size_t)r * (size_t)(cols / (32 / bits));
    uint32_t p = sb[(size_t)r * (size_t)(cols / ORACLE_GROUP) + (size_t)(c / ORACLE_GROUP)];
    double scale = bf16_value((uint16_t)(p & 0xFFFFu));
    double bias = bf16_value((uint16_t)(p >> 16));
    return (double)code_of(row, c, bits) * scale + bias;
}

double oracle_bf16_to_f64(uint16_t bits) { return bf16_value(bits); }

/* ------------------------------------------------------------------ */
/* record format                                                        */
/* ------------------------------------------------------------------ */
static size_t up256(size_t n) { return (n + 255u) / 256u * 256u; }

typedef struct {
    size_t gate_codes, up_codes, down_codes, gate_sb, up_sb, down_sb, total;
} oracle_layout;

static oracle_layout layout_of(int hidden, int inter, int bits)
{
    oracle_layout L;
    size_t gc = (size_t)inter * hidden * bits / 8;
    size_t dc = (size_t)hidden * inter * bits / 8;
    size_t gs = (size_t)inter * (hidden / ORACLE_GROUP) * 4;
    size_t ds = (size_t)hidden * (inter / ORACLE_GROUP) * 4;
    L.gate_codes = 0;
    L.up_codes = L.gate_codes + up256(gc);
    L.down_codes = L.up_codes + up256(gc);
    L.gate_sb = L.down_codes + up256(dc);
    L.up_sb = L.gate_sb + up256(gs);
    L.down_sb = L.up_sb + up256(gs);
    L.total = L.down_sb + up256(ds);
    return L;
}

/* Bytes of one expert record (gate, up, down codes + their scale/bias). */
size_t oracle_record_bytes(int hidden, int inter, int bits)
{
    return layout_of(hidden, inter, bits).total;
}

/* ------------------------------------------------------------------ */
/* dequantised matrix-vector product                                    */
/* ------------------------------------------------------------------ */
/* y[r] = sum_{c ascending} (q[r][c]*s[r][c/64] + b[r][c/64]) * x[c]
 * [openclawradar] "Metal compute shaders": 4-bit and 2-bit dequant matvec. */
void oracle_qmatvec(const uint32_t *codes, const uint32_t *sb, int rows,
                    int cols, int bits, const double *x, double *y)
{
    int r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        double acc = 0.0;
        for (int c = 0; c < cols; ++c)
            acc += dequant(codes, sb, cols, bits, r, c) * x[c];
        y[r] = acc;
    }
}

/* Materialise W[rows][cols] in fp64 (small shapes; used by the self-checks). */
void oracle_dequant_matrix(const uint32_t *codes, const uint32_t *sb, int rows,
                           int cols, int bits, double *w)
{
    for (int r = 0; r < rows; ++r)
        for (int c = 0; c < cols; ++c)
            w[(size_t)r * cols + c] = dequant(codes, sb, cols, bits, r, c);
}

/* ------------------------------------------------------------------ */
/* router, softmax, top-K                                               */
/* ------------------------------------------------------------------ */
/* logits[e] = sum_c W_r[e][c] x[c]; W_r stored expert-major [E][H] as fp32
 * (dtype 0) or bf16 bit patterns (dtype 1).
 * [openclawradar] "Pipeline performance": routing runs inside CMD2. */
void oracle_router(int dtype, const void *w, int n_experts, int hidden,
                   const double *x, double *logits)
{
    int e;
#pragma omp parallel for schedule(static)
    for (e = 0; e < n_experts; ++e) {
        double acc = 0.0;
        for (int c = 0; c < hidden; ++c) {
            size_t i = (size_t)e * hidden + c;
            double we = dtype == 0 ? (double)((const float *)w)[i]
                                   : bf16_value(((const uint16_t *)w)[i]);
            acc += we * x[c];
        }
        logits[e] = acc;
    }
}

/* p = softmax(logits), max-subtracted.
 * [openclawradar] "Pipeline performance": softmax + topK routing. */
void oracle_softmax(const double *logits, int n, double *p)
{
    double m = logits[0];
    for (int i = 1; i < n; ++i)
        if (logits[i] > m) m = logits[i];
    double z = 0.0;
    for (int i = 0; i < n; ++i) {
        p[i] = exp(logits[i] - m);
        z += p[i];
    }
    for (int i = 0; i < n; ++i) p[i] /= z;
}

/* The K largest logits, ties to the lower index, in descending order: K
 * selection passes over the experts not yet taken. */
void oracle_topk(const double *logits, int n, int k, int32_t *idx)
{
    unsigned char *taken = (unsigned char *)calloc((size_t)n, 1);
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int i = 0; i < n; ++i) {
            if (taken[i]) continue;
            if (best < 0 || logits[i] > logits[best]) best = i;
        }
        taken[best] = 1;
        idx[j] = best;
    }
    free(taken);
}

/* w[k] = p[idx[k]], divided by their sum when renorm != 0. */
void oracle_topk_weights(const double *p, const int32_t *idx, int k,
                         int renorm, double *w)
{
    double s = 0.0;
    for (int j = 0; j < k; ++j) {
        w[j] = p[idx[j]];
        s += w[j];
    }
    if (renorm)
        for (int j = 0; j < k; ++j) w[j] /= s;
}

/* sigma = 1 / (1 + exp(-(g . x))): scalar sigmoid gate of the shared expert.
 * [openclawradar] "Metal compute shaders": MoE combine + residual + sigmoid
 * gate. */
double oracle_shared_gate(int dtype, const void *g, int hidden, const double *x)
{
    double acc = 0.0;
    for (int c = 0; c < hidden; ++c) {
        double gc = dtype == 0 ? (double)((const float *)g)[c]
                               : bf16_value(((const uint16_t *)g)[c]);
        acc += gc * x[c];
    }
    return 1.0 / (1.0 + exp(-acc));
}

/* ------------------------------------------------------------------ */
/* one expert                                                            */
/* ------------------------------------------------------------------ */
/* a = W_gate x, u = W_up x, h = silu(a) * u, y = W_down h.
 * [openclawradar] "Metal compute shaders": fused SwiGLU activation. */
void oracle_expert(const uint8_t *record, int hidden, int inter, int bits,
                   const double *x, double *h, double *y)
{
    oracle_layout L = layout_of(hidden, inter, bits);
    double *a = (double *)malloc(sizeof(double) * (size_t)inter);
    double *u = (double *)malloc(sizeof(double) * (size_t)inter);
    oracle_qmatvec((const uint32_t *)(record + L.gate_codes),
                   (const uint32_t *)(record + L.gate_sb), inter, hidden, bits, x, a);
    oracle_qmatvec((const uint32_t *)(record + L.up_codes),
                   (const uint32_t *)(record + L.up_sb), inter, hidden, bits, x, u);
    for (int r = 0; r < inter; ++r) {
        double sig = 1.0 / (1.0 + exp(-a[r]));
        h[r] = a[r] * sig * u[r];
    }
    oracle_qmatvec((const uint32_t *)(record + L.down_codes),
                   (const uint32_t *)(record + L.down_sb), hidden, inter, bits, h, y);
    free(a);
    free(u);
}

/* out[o] = h_res[o] + sum_k w[k] y[k][o] + sigma * y_shared[o]
 * [openclawradar] "Metal compute shaders": combine + residual + sigmoid gate
 * in one pass. */
void oracle_combine(int hidden, int k, const double *h_res, const double *y,
                    const double *w, const double *y_shared, double sigma,
                    double *out)
{
    for (int o = 0; o < hidden; ++o) {
        double acc = h_res[o];
        for (int j = 0; j < k; ++j) acc += w[j] * y[(size_t)j * hidden + o];
        acc += sigma * y_shared[o];
        out[o] = acc;
    }
}

/* x = h / sqrt(mean(h^2) + eps): two passes, unit weight.
 * [openclawradar] "Metal compute shaders": RMS normalisation in two passes
 * (sum of squares, then apply). */
void oracle_rmsnorm(const double *h, int n, double eps, double *x)
{
    double ss = 0.0;
    for (int i = 0; i < n; ++i) ss += h[i] * h[i];
    double r = 1.0 / sqrt(ss / (double)n + eps);
    for (int i = 0; i < n; ++i) x[i] = h[i] * r;
}

/* ------------------------------------------------------------------ */
/* one MoE layer for one token                                          */
/* ------------------------------------------------------------------ */
/* Router -> softmax -> top-K -> K routed experts + the shared expert ->
 * combine.  `experts` holds n_experts records at `expert_stride` bytes.
 * Outputs (all caller-allocated): logits[E], p[E], idx[K], w[K], *sigma,
 * h[(K+1)][I] (routed in idx order, then shared), y[(K+1)][H], out[H]. */
void oracle_layer(int hidden, int inter, int n_experts, int top_k,
                  int bits_routed, int bits_shared, int renorm,
                  int router_dtype, const void *router,
                  int gate_dtype, const void *gate_vec,
                  const uint8_t *experts, size_t expert_stride,
                  const uint8_t *shared_record,
                  const double *x, const double *h_res,
                  double *logits, double *p, int32_t *idx, double *w,
                  double *sigma, double *h, double *y, double *out)
{
    oracle_router(router_dtype, router, n_experts, hidden, x, logits);
    oracle_softmax(logits, n_experts, p);
    oracle_topk(logits, n_experts, top_k, idx);
    oracle_topk_weights(p, idx, top_k, renorm, w);
    *sigma = oracle_shared_gate(gate_dtype, gate_vec, hidden, x);
    for (int j = 0; j < top_k; ++j)
        oracle_expert(experts + (size_t)idx[j] * expert_stride, hidden, inter,
                      bits_routed, x, h + (size_t)j * inter, y + (size_t)j * hidden);
    oracle_expert(shared_record, hidden, inter, bits_shared, x,
                  h + (size_t)top_k * inter, y + (size_t)top_k * hidden);
    oracle_combine(hidden, top_k, h_res, y, w, y + (size_t)top_k * hidden,
                   *sigma, out);
}

/* ------------------------------------------------------------------ */
/* gated delta-rule decode step (the linear-attention layers)          */
/* ------------------------------------------------------------------ */
/* [openclawradar] "Accelerate BLAS for linear attention" and [a2a-fr]
 * "Technical deep dive / 4": each of the 64 heads keeps a 128x128 state
 * matrix that the decode step updates with a scale (sscal), a matrix-vector
 * product (sgemv) and a rank-1 update (sger).  Taken in that order, with the
 * state S stored as d_v rows of d_k columns:
 *     S <- alpha S;  u = S k;  S <- S + beta (v - u) k^T;  o = S q
 * for every sequence and head (q, k: d_k; v, o: d_v; alpha, beta: scalars).
 * The state is updated in place. */
void oracle_gdn_step(int n_seq, int n_heads, int d_k, int d_v, const double *q,
                     const double *k, const double *v, const double *alpha,
                     const double *beta, double *state, double *out)
{
    for (int s = 0; s < n_seq; ++s) {
        for (int h = 0; h < n_heads; ++h) {
            const size_t sh = (size_t)s * n_heads + h;
            double *S = state + sh * (size_t)d_v * d_k;
            const double *qh = q + sh * d_k, *kh = k + sh * d_k, *vh = v + sh * d_v;
            double *oh = out + sh * d_v;
            const double a = alpha[sh], b = beta[sh];
            /* sscal */
            for (size_t i = 0; i < (size_t)d_v * d_k; ++i) S[i] *= a;
            for (int i = 0; i < d_v; ++i) {
                double *row = S + (size_t)i * d_k;
                /* sgemv: u_i = sum_j S_ij k_j */
                double u = 0.0;
                for (int j = 0; j < d_k; ++j) u += row[j] * kh[j];
                /* sger: S_ij += beta (v_i - u_i) k_j */
                const double c = b * (vh[i] - u);
                for (int j = 0; j < d_k; ++j) row[j] += c * kh[j];
            }
            /* sgemv: o_i = sum_j S_ij q_j */
            for (int i = 0; i < d_v; ++i) {
                const double *row = S + (size_t)i * d_k;
                double o = 0.0;
                for (int j = 0; j < d_k; ++j) o += row[j] * qh[j];
                oh[i] = o;
            }
        }
    }
}

/* ------------------------------------------------------------------ */
/* linear-attention block around the decode step                       */
/* ------------------------------------------------------------------ */
/* One gated-delta-rule block for one token ([openclawradar] "Pipeline
 * performance": CMD1 runs the attention projections and the delta net;
 * "Accelerate BLAS for linear attention": 64 heads, a 128x128 state each).
 * D = n_heads * d_head.  The projections are quantised [rows][cols]
 * matrices in two records of the expert format (hidden = H, inter = D):
 *   rec_qko: gate = W_q [D][H], up = W_k [D][H], down = W_o [H][D]
 *   rec_vab: gate = W_v [D][H], up rows 0..n_heads-1 = W_alpha,
 *            rows n_heads..2 n_heads-1 = W_beta
 * Steps, in order:
 *   x = RMSNorm(h);  q = W_q x;  k = W_k x;  v = W_v x;
 *   a = W_alpha x;  b = W_beta x;
 *   per head: q_h /= sqrt(|q_h|^2 + 1e-6);  k_h /= sqrt(|k_h|^2 + 1e-6);
 *             alpha_h = 1 / (1 + exp(-a_h));  beta_h = 1 / (1 + exp(-b_h));
 *   the decode step of every head on `state` ([n_heads][d_head][d_head],
 *   updated in place) -> o [D];
 *   h_out = h + W_o o.
 * Also returns the projections (proj: q, k, v as projected, then a, b) and
 * o, for per-stage checks.  proj holds 3 D + 2 n_heads values. */
void oracle_gdn_block(int hidden, int n_heads, int d_head, int bits,
                      const uint8_t *rec_qko, const uint8_t *rec_vab,
                      const double *h, double *state, double *proj,
                      double *o, double *h_out)
{
    const int D = n_heads * d_head;
    const oracle_layout lay = layout_of(hidden, D, bits);
    double *x = (double *)malloc(sizeof(double) * (size_t)hidden);
    double *q = (double *)malloc(sizeof(double) * (size_t)D);
    double *k = (double *)malloc(sizeof(double) * (size_t)D);
    double *alpha = (double *)malloc(sizeof(double) * (size_t)n_heads);
    double *beta = (double *)malloc(sizeof(double) * (size_t)n_heads);
    double *y = (double *)malloc(sizeof(double) * (size_t)hidden);
    oracle_rmsnorm(h, hidden, 1e-6, x);
    oracle_qmatvec((const uint32_t *)(rec_qko + lay.gate_codes),
                   (const uint32_t *)(rec_qko + lay.gate_sb), D, hidden, bits, x, proj);
    oracle_qmatvec((const uint32_t *)(rec_qko + lay.up_codes),
                   (const uint32_t *)(rec_qko + lay.up_sb), D, hidden, bits, x, proj + D);
    oracle_qmatvec((const uint32_t *)(rec_vab + lay.gate_codes),
                   (const uint32_t *)(rec_vab + lay.gate_sb), D, hidden, bits, x, proj + 2 * D);
    oracle_qmatvec((const uint32_t *)(rec_vab + lay.up_codes),
                   (const uint32_t *)(rec_vab + lay.up_sb), 2 * n_heads, hidden, bits, x,
                   proj + 3 * D);
    for (int hd = 0; hd < n_heads; ++hd) {
        const double *qh = proj + (size_t)hd * d_head;
        const double *kh = proj + D + (size_t)hd * d_head;
        double nq = 0.0, nk = 0.0;
        for (int j = 0; j < d_head; ++j) nq += qh[j] * qh[j];
        for (int j = 0; j < d_head; ++j) nk += kh[j] * kh[j];
        const double rq = 1.0 / sqrt(nq + 1e-6), rk = 1.0 / sqrt(nk + 1e-6);
        for (int j = 0; j < d_head; ++j) {
            q[(size_t)hd * d_head + j] = qh[j] * rq;
            k[(size_t)hd * d_head + j] = kh[j] * rk;
        }
        alpha[hd] = 1.0 / (1.0 + exp(-proj[3 * D + hd]));
        beta[hd] = 1.0 / (1.0 + exp(-proj[3 * D + n_heads + hd]));
    }
    oracle_gdn_step(1, n_heads, d_head, d_head, q, k, proj + 2 * D, alpha, beta, state, o);
    oracle_qmatvec((const uint32_t *)(rec_qko + lay.down_codes),
                   (const uint32_t *)(rec_qko + lay.down_sb), hidden, D, bits, o, y);
    for (int i = 0; i < hidden; ++i) h_out[i] = h[i] + y[i];
    free(x); free(q); free(k); free(alpha); free(beta); free(y);
}
