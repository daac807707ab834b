/*
 * moe.h -- C ABI of libmoe, the MI355X (gfx950) MoE expert hot path.
 *
 * One MoE layer for one token (or a micro-batch of tokens):
 *   router matvec -> softmax -> top-K of E experts -> for the K routed experts
 *   and one shared expert a groupwise-affine 4-bit or 2-bit dequantised matvec
 *   (w = q * scale + bias) for gate and up, fused SwiGLU, the down matvec, and
 *   a weighted combine with a sigmoid-gated shared expert plus the residual.
 *
 * The operations follow these pages (cited by site and section):
 *   [openclawradar] openclawradar.com (ja), "Flash-MoE: running the 397B
 *       parameter Qwen model on a MacBook Pro in pure C/Metal": "Technical
 *       implementation" (hidden 4096, 512 experts, K=4 plus one shared),
 *       "FMA-optimized dequant kernel", "Metal compute shaders" (4/2-bit
 *       dequant matvec, fused SwiGLU, two-pass RMSNorm, combine + residual +
 *       sigmoid gate), "Deferred GPU expert compute", "Pipeline performance"
 *       (softmax + topK routing).
 *   [a2a-fr] a2a-mcp.org (fr), "What is Flash-MoE?": "FMA-optimised
 *       dequantisation kernels" (nibble * scale + bias).
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees, copies between host and device, or synchronises
 *     in these calls, so every call may be captured into a HIP graph.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *   - Arguments are checked before anything is enqueued.  On failure the call
 *     returns a negative status, enqueues nothing and leaves a message for
 *     moe_last_error() (thread-local).  A failed kernel launch returns
 *     MOE_EHIP with the HIP error string.  Faults inside kernels surface at the
 *     caller's next stream synchronisation.
 *   - Environment: MOE_DEBUG=1 makes every call synchronise its stream after
 *     each launch made outside stream capture and return MOE_EHIP for a
 *     launch that faulted (triage only: it breaks the no-synchronisation
 *     rule above).  MOE_TUNE="gu=<p>,dn=<p>,sh=<p>" (p = 1, 2 or 4) overrides
 *     the rows a wave takes per pass in the gate/up, down and shared kernels.
 *   - Kernels never read outside the buffers described here.  An expert id
 *     that is neither in [0, n_experts) nor MOE_SHARED yields a NaN row.
 *   - Limits: bits 4 or 2, group 64 (else MOE_EUNSUPPORTED); hidden and inter
 *     multiples of 64 in [64, 8192]; 1 <= top_k <= 8, top_k <= n_experts <=
 *     1024; 1 <= n_tokens <= 64.  Alignment: records, expert_stride and the
 *     workspace on 256 bytes, every other vector on 16 bytes (MOE_EALIGN).
 *   - Reentrant: the only global state is thread-local (the error string and
 *     the kernel-timing switch of moe_profile_begin).
 *
 * Record format (one expert, `moe_expert_bytes` bytes, sections on 256-byte
 * boundaries, in this order):
 *   codes_gate [inter][hidden*bits/32] u32, codes_up [inter][hidden*bits/32],
 *   codes_down [hidden][inter*bits/32], sb_gate [inter][hidden/64] u32,
 *   sb_up [inter][hidden/64], sb_down [hidden][inter/64].
 *   Codes are unsigned b-bit fields, little-endian in each 32-bit word: column
 *   c of a row sits in word c*b/32 at bit b*(c mod 32/b).  Each sb word holds
 *   the bf16 scale (low 16 bits) and bf16 bias (high 16 bits) of 64
 *   consecutive input columns.  The dequantised weight is q*scale + bias with
 *   no zero point ([a2a-fr] "FMA-optimised dequantisation kernels").
 *   At hidden 4096 / inter 1024 / 4 bits a record is 7,077,888 bytes = 6.75
 *   MiB, the "about 6.75 MB per expert" of [openclawradar] "SSD expert
 *   streaming".
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,        /* null pointer, bad size or count */
    MOE_EUNSUPPORTED = -2,  /* bits, group or dtype outside what is built */
    MOE_EALIGN = -3,        /* pointer or stride misaligned */
    MOE_EWORKSPACE = -4,    /* workspace missing or too small */
    MOE_EHIP = -5           /* a HIP runtime call failed */
};

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* expert id that selects the layer's shared expert in an id list */
#define MOE_SHARED (-1)

/* One MoE layer: shapes, flags and device pointers to its weights.  A host
 * struct, read by the callee only during the call. */
typedef struct moe_layer {
    int hidden;            /* H: model width */
    int inter;             /* I: expert intermediate width (routed and shared) */
    int n_experts;         /* E: routed experts */
    int top_k;             /* K: routed experts per token */
    int group;             /* quantisation group along the input dim; must be 64 */
    int bits_routed;       /* 4 or 2 */
    int bits_shared;       /* 4 or 2 */
    int renorm_topk;       /* 1: the K selected probabilities are divided by
                              their sum; 0: they are the plain softmax values */
    moe_dtype router_dtype;
    const void *router;    /* [E][H] router weights, expert-major */
    moe_dtype gate_dtype;
    const void *shared_gate;   /* [H] shared-expert gate vector g */
    const void *experts;       /* E routed records, `expert_stride` bytes apart */
    size_t expert_stride;
    const void *shared_expert; /* one record at bits_shared */
    const void *router_tiles;  /* optional (may be NULL): the router re-laid by
                                  moe_router_tile; stacks then read it to form
                                  each layer's routing sums (same values,
                                  coalesced reads).  16-byte aligned. */
} moe_layer_t;

/* ---------------------------------------------------------------------- */
/* status, sizes                                                           */
/* ---------------------------------------------------------------------- */
const char *moe_strerror(int status);
/* Detail of the last failure on this thread ("" if none). */
const char *moe_last_error(void);
/* ABI version of this header (increments on incompatible change). */
int moe_abi_version(void);

/* Bytes of one quantised [rows][cols] matrix: codes plus sb words, each
 * section rounded up to 256 bytes ([a2a-fr] "FMA-optimised dequantisation
 * kernels": b-bit codes with a scale and a bias per group of inputs).  0 when
 * the shape is invalid. */
size_t moe_qmatrix_bytes(int rows, int cols, int bits, int group);
/* Bytes of one expert record (see the format above).  0 when invalid. */
size_t moe_expert_bytes(int hidden, int inter, int bits, int group);
/* Byte offsets of the six sections of a record, in record order:
 * codes_gate, codes_up, codes_down, sb_gate, sb_up, sb_down. */
int moe_expert_offsets(int hidden, int inter, int bits, int group, size_t out[6]);
/* Workspace bytes that moe_layer_decode / moe_route / moe_expert_forward_*
 * need for this layer and token count (0 if the layer is invalid): the
 * intermediates that [openclawradar] "Deferred GPU expert compute" keeps on
 * the device between the routing and the expert pass (logits, gate sigma,
 * SwiGLU outputs, the shared expert's output). */
size_t moe_layer_workspace_bytes(const moe_layer_t *L, int n_tokens);
/* Workspace bytes moe_stack_decode needs for `n_layers` layers shaped like L. */
size_t moe_stack_workspace_bytes(const moe_layer_t *L, int n_layers);

/* ---------------------------------------------------------------------- */
/* the path, stage by stage                                                 */
/* ---------------------------------------------------------------------- */
/* Router matvec, softmax, top-K and the shared sigmoid gate for n_tokens
 * tokens ([openclawradar] "Pipeline performance": routing, then softmax +
 * topK).
 *   x            [n_tokens][H], x_dtype
 *   topk_idx     [n_tokens][K] int32: the K largest logits, exact ties to the
 *                lower expert index, in descending order
 *   topk_w       [n_tokens][K] fp32: softmax probabilities of those experts
 *                (renormalised to sum 1 when L->renorm_topk)
 *   shared_sigma [n_tokens] fp32: 1 / (1 + exp(-(g . x)))
 *   logits       [n_tokens][E] fp32, or NULL (16-byte aligned: the top-K
 *                kernel reads it with 16-byte loads)
 *   ws           workspace of moe_layer_workspace_bytes(L, n_tokens) bytes */
int moe_route(const moe_layer_t *L, int n_tokens, moe_dtype x_dtype, const void *x,
              int32_t *topk_idx, float *topk_w, float *shared_sigma, float *logits,
              void *ws, size_t ws_bytes, void *stream);

/* Expert forward for a list of experts on one token: for each listed id e,
 *   h_e = silu(W_gate(e) x) * (W_up(e) x)   [I]   (fused SwiGLU)
 *   y_e = W_down(e) h_e                      [H]
 * with every W the dequantised q*scale + bias matrix ([openclawradar]
 * "FMA-optimized dequant kernel", "Metal compute shaders").
 *   expert_ids  [n] int32 device array; MOE_SHARED selects the shared record
 *   y           [n][H] fp32 output
 *   h           [n][I] fp32 output, or NULL (then kept in the workspace)
 * The _q4 entry point needs L->bits_routed == 4, the _q2 entry point
 * L->bits_routed == 2; a MOE_SHARED entry whose bits_shared differs from the
 * entry point's width yields a NaN row.  1 <= n <= 64. */
int moe_expert_forward_q4(const moe_layer_t *L, moe_dtype x_dtype, const void *x,
                          const int32_t *expert_ids, int n, float *y, float *h,
                          void *ws, size_t ws_bytes, void *stream);
int moe_expert_forward_q2(const moe_layer_t *L, moe_dtype x_dtype, const void *x,
                          const int32_t *expert_ids, int n, float *y, float *h,
                          void *ws, size_t ws_bytes, void *stream);

/* out[o] = h_res[o] + sum_k w[k] * y[k][o] + shared_sigma[0] * y_shared[o]
 * ([openclawradar] "Metal compute shaders": MoE combine + residual + sigmoid
 * gate in one pass).  y is [n_routed][hidden]; every array fp32.  h_out may
 * alias h_res. */
int moe_combine(int hidden, int n_routed, const float *h_res, const float *y,
                const float *w, const float *y_shared, const float *shared_sigma,
                float *h_out, void *stream);

/* ---------------------------------------------------------------------- */
/* whole layer, whole stack                                                 */
/* ---------------------------------------------------------------------- */
/* One MoE layer for n_tokens tokens with no host round trip: routing, the K
 * routed experts and the shared expert, combine + residual ([openclawradar]
 * "Pipeline performance": routing (softmax + topK) then the expert forward,
 * combine and norm of one layer; "Deferred GPU expert compute": the expert
 * pass is queued on the GPU without a host wait).
 *   x        [n_tokens][H] (x_dtype), the normalised activation
 *   h_res    [n_tokens][H] fp32 residual; h_out [n_tokens][H] fp32 (may not
 *            alias h_res)
 *   topk_idx [n_tokens][K], topk_w [n_tokens][K]: the routing decision
 * Intermediates (logits, sigma, h_e, the shared expert's y) stay in `ws`; see
 * moe_layer_ws_view. */
int moe_layer_decode(const moe_layer_t *L, int n_tokens, moe_dtype x_dtype, const void *x,
                     const float *h_res, float *h_out, int32_t *topk_idx, float *topk_w,
                     void *ws, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * moe_layer_decode with its workspace in a library-owned device array of
 * MOE_NOALLOC_SCRATCH_BYTES per GPU instead of a caller's buffer.  The call
 * allocates nothing.  The array lives until the process ends; the first call
 * on a device looks up its address there (make that first call outside a
 * graph capture).  A layer and token count whose workspace
 * (moe_layer_workspace_bytes) exceeds the array are refused with
 * MOE_EWORKSPACE before anything is enqueued; the q4 layer needs about 0.3
 * MiB for one token and 1.7 MiB for 16.  Every call on one GPU shares its
 * array and leaves its intermediates there (nothing in it has to start at
 * zero): calls that overlap in time on one GPU, on different streams or
 * from different threads, race. */
#define MOE_NOALLOC_SCRATCH_BYTES (8u << 20)
int moe_layer_decode_noalloc(const moe_layer_t *L, int n_tokens, moe_dtype x_dtype,
                             const void *x, const float *h_res, float *h_out,
                             int32_t *topk_idx, float *topk_w, void *stream);

/* Device pointers of the intermediates moe_layer_decode leaves in ws. */
typedef struct moe_ws_view {
    float *logits;       /* [n_tokens][E] */
    float *sigma;        /* [n_tokens] */
    float *h_routed;     /* [n_tokens][K][I] routed SwiGLU outputs, idx order */
    float *h_shared;     /* [n_tokens][I] shared SwiGLU output */
} moe_ws_view;
int moe_layer_ws_view(const moe_layer_t *L, int n_tokens, void *ws, size_t ws_bytes,
                      moe_ws_view *view);

/* One token through n_layers layers, residual carried in fp32:
 *   for l: h <- h + u_l (u_l = updates_bf16[l], skipped when NULL);
 *          x = h / sqrt(mean(h^2) + 1e-6)  (two-pass RMSNorm, unit weight,
 *          [openclawradar] "Metal compute shaders");
 *          h <- h + MoE_l(x)   (moe_layer_decode with h_res = h)
 *   h       [H] fp32, read and overwritten
 *   idx_log [n_layers][K], w_log [n_layers][K]: routing of every layer
 * All layers must share hidden/inter/E/K/bits/dtypes with layers[0].
 * With bits_shared == bits_routed the router dots, gate dot and sum of
 * squares of each layer's input are summed in fp64 from fp32 partials of row
 * tiles, added in the order the tiles finish: the fp64 sum is exact unless the
 * partials of one value span more than about 2^22 in magnitude, so a logit can
 * differ in its last fp32 place between calls only with a chance of about
 * 2^-29. */
int moe_stack_decode(const moe_layer_t *layers, int n_layers, const uint16_t *updates_bf16,
                     float *h, int32_t *idx_log, float *w_log,
                     void *ws, size_t ws_bytes, void *stream);

/* The router [E][H] (dtype router_dtype) re-laid for stacks as column tiles:
 * out[t][e][j] = router[e][8 t + j] for t < H / 8, j < 8, so that the eight
 * columns of every expert in a tile are one 16-byte (bf16) or 32-byte (fp32)
 * run and the experts of a tile are consecutive.  A stack layer's combine
 * reads, for its rows, one such run per expert of the next layer: the router
 * slices of [openclawradar] "Pipeline performance" CMD3 (combine + norm
 * feeding the next layer's routing), read without strided row accesses.
 * out: E * H * element bytes, 16-byte aligned, caller-owned, not aliasing
 * router.  H must be a multiple of 64.  Enqueued on `stream`. */
int moe_router_tile(const void *router, int n_experts, int hidden, moe_dtype router_dtype,
                    void *out, void *stream);

/* One token through a stack whose layers may open with a linear-attention
 * block ([openclawradar] "Technical implementation": 45 GatedDeltaNet
 * layers and 15 full-attention layers; "Accelerate BLAS for linear
 * attention": 64 heads, a 128x128 state each, scale + gemv + rank-1 update;
 * "Pipeline performance": CMD1 runs the attention projections and the delta
 * net).  For layer l with gdn[l].state set:
 *   x = RMSNorm(h); q = W_q x, k = W_k x, v = W_v x (n_heads x d_head each),
 *   a = W_alpha x, b = W_beta x (one per head); per head q and k scaled to
 *   unit length (q / sqrt(|q|^2 + 1e-6)), alpha = sigmoid(a), beta =
 *   sigmoid(b); then S <- alpha S, u = S k, S <- S + beta (v - u) k^T,
 *   o = S q on the layer's state (updated in place); h <- h + W_o o;
 * otherwise h <- h + u_l (updates_bf16 row l, skipped when NULL), the stand-in
 * for a full-attention layer.  Then the MoE layer of moe_stack_decode.  The
 * projections are quantised matrices in two records of the expert format
 * with hidden = H and inter = D = n_heads * d_head (moe_expert_bytes(H, D,
 * bits) bytes each, 256-byte aligned):
 *   rec_qko: gate = W_q [D][H], up = W_k [D][H], down = W_o [H][D]
 *   rec_vab: gate = W_v [D][H], up rows 0..n_heads-1 = W_alpha,
 *            rows n_heads..2 n_heads-1 = W_beta (the other rows unused)
 * d_head in {16, 32, 64, 128, 256}, D a multiple of 64 up to 8192; state
 * [n_heads][d_head][d_head] fp32 (row i of a head's state is value i).
 * ws: moe_stack_gdn_workspace_bytes bytes. */
typedef struct moe_gdn_layer {
    int n_heads, d_head, bits;
    const void *rec_qko;
    const void *rec_vab;
    float *state;          /* NULL: a full-attention layer (the update is used) */
} moe_gdn_layer_t;
size_t moe_stack_gdn_workspace_bytes(const moe_layer_t *L, const moe_gdn_layer_t *gdn, int n_layers);
int moe_stack_decode_gdn(const moe_layer_t *layers, const moe_gdn_layer_t *gdn, int n_layers,
                         const uint16_t *updates_bf16, float *h, int32_t *idx_log, float *w_log,
                         void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------- */
/* host-memory expert tier ([openclawradar] "SSD expert streaming",         */
/* "Pipeline performance" and "Architecture constraint"; [a2a-fr] "Technical */
/* deep dive / 1": only the routed experts of a token are read, on demand,   */
/* after the routing, and a cache (the OS page cache on the pages) serves    */
/* repeats)                                                                  */
/* ---------------------------------------------------------------------- */
typedef struct moe_tier_s *moe_tier_t;
/* Device bytes of a tier's state: a tick, the hit / miss / byte counters and
 * the owner and last use of every slot (0 for invalid sizes). */
size_t moe_tier_state_bytes(int n_experts, int n_slots);
/* A cache of n_slots routed-expert records in device memory in front of all
 * E records of one layer in host memory, managed on the device.
 *   host_records  E records, expert_stride bytes apart, caller-owned
 *                 page-locked host memory the device can read (hipHostMalloc;
 *                 a pinned torch tensor); MOE_EINVAL for pageable memory
 *   cache         n_slots x expert_stride bytes of device memory
 *   state         moe_tier_state_bytes(E, n_slots) bytes of device memory;
 *                 moe_tier_reset initialises it before the first decode
 * All caller-owned, 256-byte aligned, outliving the tier.  K <= 8 <= n_slots
 * <= E <= 1024.  The handle holds the pointers and shapes (host memory, no
 * device memory is allocated).  One stream at a time may use a tier. */
int moe_tier_create(const void *host_records, int n_experts, size_t expert_stride,
                    void *cache, int n_slots, void *state, moe_tier_t *out);
int moe_tier_destroy(moe_tier_t t);
/* Empty the cache and zero the counters (a kernel on `stream`). */
int moe_tier_reset(moe_tier_t t, void *stream);
/* moe_layer_decode for one token with the routed experts read through the
 * tier, entirely on the device (no host wait; the call can be captured into
 * a graph): the router, then one kernel that takes the top K and gives each
 * selected expert its slot -- the slot holding it (a hit), else the least
 * recently used slot this token has not taken (never-used slots first, the
 * lowest slot among equal uses) -- then the gate/up launch, which reads a
 * hit's gate/up rows from its slot and a miss's straight from host memory,
 * writing them into the slot as it reads them, while extra workgroups of the
 * same launch copy each miss's down rows from host memory into its slot;
 * then down + combine on the slots.  A miss therefore crosses the host link
 * once, and its transfer overlaps the hits' and the shared expert's work.
 * L->experts and L->expert_stride are not used.  The outputs (topk_idx holds
 * expert ids) equal those of moe_layer_decode. */
int moe_tier_layer_decode(const moe_layer_t *L, moe_tier_t t, moe_dtype x_dtype, const void *x,
                          const float *h_res, float *h_out, int32_t *topk_idx, float *topk_w,
                          void *ws, size_t ws_bytes, void *stream);
/* Hits, misses and record bytes read from host memory since the last reset,
 * and (if slot_owner is not NULL) the expert in each slot ([n_slots], -1 for
 * an empty slot); any output may be NULL.  A query outside the decode path:
 * it copies the state to the host and waits for `stream`. */
int moe_tier_stats(moe_tier_t t, void *stream, unsigned long long *hits,
                   unsigned long long *misses, unsigned long long *bytes_read,
                   int32_t *slot_owner);

/* ---------------------------------------------------------------------- */
/* HIP graphs ([openclawradar] "Deferred GPU expert compute": the expert     */
/* pass is queued without a host wait)                                      */
/* ---------------------------------------------------------------------- */
typedef struct moe_graph_s *moe_graph_t;
/* Start capturing every call made on `stream` (which must not be the NULL
 * stream) into a graph; end and instantiate it with moe_graph_capture_end. */
int moe_graph_capture_begin(void *stream);
int moe_graph_capture_end(void *stream, moe_graph_t *out);
/* Capture moe_stack_decode with these arguments (the buffers must outlive
 * the graph). */
int moe_graph_create_stack(const moe_layer_t *layers, int n_layers,
                           const uint16_t *updates_bf16, float *h, int32_t *idx_log,
                           float *w_log, void *ws, size_t ws_bytes, void *stream,
                           moe_graph_t *out);
int moe_graph_launch(moe_graph_t g, void *stream);
int moe_graph_destroy(moe_graph_t g);

/* ---------------------------------------------------------------------- */
/* kernel timing                                                            */
/* ---------------------------------------------------------------------- */
/* Kernels the library launches, as reported by moe_profile_end. */
enum {
    MOE_KERNEL_HEAD = 1,       /* router rows + shared gate + shared gate/up */
    MOE_KERNEL_GATEUP = 2,     /* routed gate/up + SwiGLU (with top-K) */
    MOE_KERNEL_DOWN = 3,       /* down projections + combine + residual */
    MOE_KERNEL_DOWN_Y = 4,     /* down projection writing per-expert y */
    MOE_KERNEL_TOPK = 5,
    MOE_KERNEL_COMBINE = 6,
    MOE_KERNEL_OTHER = 7,
    MOE_KERNEL_GDN_IN = 8,     /* linear-attention block: norm + projections */
    MOE_KERNEL_GDN_STEP = 9,   /* the gated delta-rule step */
    MOE_KERNEL_GDN_OUT = 10    /* output projection + residual */
};
/* Between moe_profile_begin and moe_profile_end, on the calling thread, every
 * kernel launch of the path entry points records two HIP events through its
 * own dispatch (hipExtLaunchKernel: the events mark the kernel's start and
 * end, with no marker packets in between), except while its stream is being
 * captured into a graph.  Up to max_launches launches are recorded; later
 * ones are not.  The events are created here and destroyed by
 * moe_profile_end.  Kernel tracers that wrap launches distort these times. */
int moe_profile_begin(int max_launches);
/* Wait for the recorded launches and write, in launch order, the elapsed
 * milliseconds between each launch's two events (ms[i]) and its kernel id
 * (kernel_ids[i], may be NULL); *n_out receives the number written. */
int moe_profile_end(float *ms, int *kernel_ids, int capacity, int *n_out);

/* ---------------------------------------------------------------------- */
/* linear-attention decode step                                             */
/* ---------------------------------------------------------------------- */
/* One gated delta-rule step for every (sequence, head) pair: the state of
 * the linear-attention layers, 64 heads of 128x128 on the pages, updated by a
 * scale, a matrix-vector product and a rank-1 update ([openclawradar]
 * "Accelerate BLAS for linear attention"; [a2a-fr] "Technical deep dive / 4").
 * With S the d_v x d_k state of one head (row-major), in this order:
 *     S <- alpha S;  u = S k;  S <- S + beta (v - u) k^T;  out = S q.
 * q, k: [n_seq][n_heads][d_k]; v, out: [n_seq][n_heads][d_v];
 * alpha, beta: [n_seq][n_heads]; state: [n_seq][n_heads][d_v][d_k] fp32,
 * updated in place.  All device pointers, fp32.  d_k must be 16, 32, 64,
 * 128 or 256 (MOE_EUNSUPPORTED otherwise), 1 <= d_v <= 8192; q, k and state
 * 16-byte aligned (MOE_EALIGN).  state may not overlap the other arrays. */
int moe_gdn_step(int n_seq, int n_heads, int d_k, int d_v, const float *q, const float *k,
                 const float *v, const float *alpha, const float *beta, float *state,
                 float *out, void *stream);

/* ---------------------------------------------------------------------- */
/* synthetic weights                                                        */
/* ---------------------------------------------------------------------- */
/* Fill n expert records at dst (stride bytes apart) with seeded synthetic
 * weights: codes uniform over 0..2^bits-1 and (scale, bias) uniform in
 * [scale_lo, scale_hi) x [bias_lo, bias_hi), rounded to bf16.  Record j gets
 * generator ids (seed, layer, first_expert + j).  The numbers come from the
 * SplitMix64 generator (Steele, Lea and Flood, OOPSLA 2014) used
 * counter-style: output i of a generator in state k is mix(k + (i+1)*GAMMA);
 * key(seed, layer, expert, section) applies that rule once per id starting
 * from the root state 0x6D6F652D67656E31.  Code words: output j fills words
 * 2j (low half) and 2j+1 (high half).  sb word i: output i, scale from its
 * bits 40..63 and bias from bits 16..39 as v = lo + (hi-lo)*((u+0.5)/2^24) in
 * fp64 without contraction, then rounded to nearest-even bf16.
 * Sections 0..5 are codes_gate, codes_up, codes_down, sb_gate, sb_up,
 * sb_down.  Padding bytes are left untouched. */
int moe_fill_experts(void *dst, size_t stride, int n, uint64_t seed, int layer,
                     int first_expert, int hidden, int inter, int bits,
                     double scale_lo, double scale_hi, double bias_lo, double bias_hi,
                     void *stream);

/* Zero `bytes` bytes at `ptr` with a kernel (no memset node, safe inside a
 * captured graph).  ptr 16-byte aligned. */
int moe_zero(void *ptr, size_t bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
