/*
 * moe_latent.h -- C ABI of the latent mixture-of-experts layer forward for
 * AMD Instinct MI355X (gfx950).
 *
 * What the layer computes (Hugging Face card "Edge0-145B . Q3_K", section
 * "Architecture", the paragraph under the architecture table, and its table
 * rows "Experts" and "Expert pool"; agentspulse tutorial "Edge0-145B hardware
 * requirements", section "latent MoE architecture"; alphasignal news, table
 * "Released model variants"):
 *
 *   h    = x D^T                   the token is projected down from the
 *                                  residual width (hidden) to the latent width
 *   l    = h R^T + b               router logits over all experts
 *   S, w = top_k(softmax(l))       the router picks k experts per token;
 *                                  weights renormalised over the chosen k
 *   z    = sum_j w_j E_{S_j}(h) + E_shared(h)
 *                                  routed SwiGLU experts latent -> inter ->
 *                                  latent, plus one shared expert alongside
 *   out  = z U^T                   the combined result projected back up
 *
 *   E_e(v) = W_down,e (silu(W_gate,e v) * (W_up,e v)),  silu(v) = v/(1+e^-v)
 *
 * The 145B layer has hidden 2560, latent 1792, 512 experts, inter 640,
 * top_k 10, one shared expert; the 120B layer has latent 1280.
 *
 * Readings where the pages are silent (they name the weight format "NVFP4"
 * and say the router "picks 10 of 512", nothing more):
 *   - gating: softmax over every expert's logit, the k largest logits (exact
 *     ties to the lower index, descending order), weights renormalised over
 *     the chosen k; no scaling factor, noise, capacity limit or dropping;
 *   - expert weights: 4-bit e2m1 codes (OCP MX v1.0), one E4M3fn block scale
 *     (OCP FP8 v1.0) per 16 consecutive input elements of one output row, one
 *     fp32 scale per matrix:  W[n][k] = e2m1(c[n][k]) * e4m3(s[n][k/16]) * g;
 *   - one D and one U per layer; the shared expert has weight 1 and the same
 *     shape and format as a routed expert;
 *   - the residual block used to stack layers is x + MoE(rmsnorm(x) * g_norm).
 *
 * Precision: bf16 matrix-core products with fp32 accumulation. The router
 * reads the latent vector at (better than) 2^-16 relative precision, so its
 * logits agree with an fp32 evaluation to about 1e-5; the experts read it
 * rounded to bf16. Expert activations and combined outputs are bf16 between
 * kernels; `out` is bf16, rounded to nearest even.
 *
 * Layouts (all row-major, innermost index contiguous; "bf16" is the upper
 * half of an IEEE binary32, passed as uint16_t; G = dims.n_groups):
 *   x, out         bf16 [T][hidden]
 *   D              bf16 [G * latent][hidden]   (D_g = rows g*latent ..)
 *   U              bf16 [hidden][G * latent]   (U_g = columns g*latent ..)
 *   router.w       bf16 [n_experts][latent];  router.bias fp32 [n_experts] or NULL
 *   fp4 matrix set of `count` matrices of shape [N][K]:
 *     codes  uint8 [count][N][K/2]   element 2j in the low nibble of byte j,
 *                                    element 2j+1 in the high nibble
 *     scales uint8 [count][N][K/16]  E4M3fn bits, block b covers k in [16b, 16b+16)
 *     gscale fp32  [count]
 *   experts.gate, experts.up: N = inter, K = latent;  experts.down: N = latent,
 *   K = inter. The shared expert uses the same layout with count 1.
 *   Mixed 3/4-bit expert record (moe_fp4_matrix.bits = 3 on gate and up;
 *   down stays e2m1). The card's Q3_K build is only partly 3-bit and keeps
 *   its experts in fixed-size records (Hugging Face card "Edge0-145B . Q3_K",
 *   section "Architecture"); no page defines the 3-bit element, so this
 *   format is this library's own. E1M1: 1 sign bit, 1 exponent bit (bias 1,
 *   exponent 0 subnormal), 1 mantissa bit, so magnitudes 0, 0.5, 1, 1.5 (the
 *   e2m1 values whose top exponent bit is clear), with the same E4M3 block
 *   scales and fp32 matrix scale as e2m1:
 *     codes  uint8 [count][N][K/32][12]   one 12-byte chunk per 32 elements,
 *            three little-endian u32 words w0, w1, w2: for g < 3, nibble p
 *            of w_g (bits 4p .. 4p+3) is element 8g + p as an e2m1 code
 *            (sign bit 3, exponent bit 1, mantissa bit 0); the nibble's
 *            bit 2, never set by an E1M1 value, holds element 24 + p: its
 *            mantissa in w0, its exponent in w1, its sign in w2
 *     scales, gscale as above.
 *   Packed copies (moe_fp4_pack / moe_bf16_pack) hold the same bytes
 *   reordered so that each wave's weight loads are contiguous 1 KB runs; a
 *   path reading them gives bit-identical results. One layout per path:
 *   grouped-packed fp4 set (N a multiple of 32, K of 64): block (e, t, s) covers
 *     matrix e, rows [32t, 32t+32), columns [64s, 64s+64); blocks are stored
 *     in (e, t, s) order, each as 64 lanes L of
 *       codes  16 bytes: row 32t + r(L % 32), columns 64s + 32(L/32) .. +32
 *              (plain byte order), at codes + 1024 * block + 16 L
 *       scales  2 bytes: the two block scales of those 32 columns,
 *              at scales + 128 * block + 2 L
 *     where r(m) = 16 (q / 8) + 8 ((m / 4) % 2) + q % 8 with
 *     q = 4 (m / 8) + m % 4 (a permutation of 0..31: it puts a matrix-core
 *     lane's results on consecutive output columns). gscale is unchanged.
 *   grouped-packed bf16 matrix [N][K] (N a multiple of 32, K of 64):
 *     block (t, s) covers rows [32t, 32t+32), columns [64s, 64s+64); blocks
 *     in (t, s) order, 4096 bytes each: the 16 bytes at 1024 q + 16 L of a
 *     block (q = 0..3, L = 0..63) are row 32t + r(L % 32), columns
 *     64s + 32(L/32) + 8q .. +8.
 *   decode-packed fp4 set (N a multiple of 16, K of 128): block (e, t, c)
 *     covers matrix e, rows [16t, 16t+16), columns [128c, 128c+128), blocks
 *     in (e, t, c) order; codes 1 KB per block, the 16 bytes at 16 l
 *     (l = 0..63) being row 16t + l % 16, columns 128c + 32(l/16) .. +32;
 *     scales 128 bytes per block, row 16t + i's eight block scales of the
 *     128 columns at 8 i.
 *   E1M1 sets pack the same way with each lane's 32 columns as one 12-byte
 *     chunk instead of 16 bytes: grouped blocks are 768 bytes of codes, lane
 *     L's chunk at 12 L; decode blocks 768 bytes, lane l's chunk at 12 l.
 *     Scales are packed as for e2m1.
 *   decode-packed bf16 matrix [N][K] (N a multiple of 16, K of 32): block
 *     (t, c) covers rows [16t, 16t+16), columns [32c, 32c+32), blocks in
 *     (t, c) order, 1 KB each, the 16 bytes at 16 l being row 16t + l % 16,
 *     columns 32c + 8(l/16) .. +8.
 *
 * Ownership: the caller allocates every buffer (device memory) and owns it.
 * Calls never allocate or free device memory and keep no pointer after they
 * return; buffers must stay valid until the work enqueued on `stream`
 * completes. Concurrent calls must not share a workspace.
 *
 * Errors: 0 on success, else a negative code. Every argument is validated
 * before anything is enqueued, so an error return leaves the device
 * untouched (except MOE_LATENT_EHIP, returned when a launch fails).
 * moe_latent_last_error() describes the last error of the calling thread.
 * Faults inside kernels surface at the caller's next synchronisation.
 */
#ifndef MOE_LATENT_H
#define MOE_LATENT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_LATENT_ABI_VERSION 4

#define MOE_LATENT_OK 0
#define MOE_LATENT_EINVAL (-1)       /* null pointer, bad size, misaligned pointer, aliasing */
#define MOE_LATENT_EUNSUPPORTED (-2) /* dims outside what the kernels handle */
#define MOE_LATENT_EWORKSPACE (-3)   /* workspace smaller than moe_latent_workspace_bytes() */
#define MOE_LATENT_EHIP (-4)         /* a HIP launch failed; message in last_error */

/* Supported dims: hidden, latent, inter positive multiples of 32;
 * 1 <= n_experts <= 1024; 1 <= top_k <= min(16, n_experts);
 * n_shared in {0, 1}; n_groups 0 or 1 (one D/U pair) or G > 1 dividing
 * n_experts; T * top_k < 2^31. */
typedef struct moe_latent_dims {
  int32_t hidden;    /* residual width (2560) */
  int32_t latent;    /* latent width (1792 for 145B, 1280 for 120B) */
  int32_t n_experts; /* routed experts per layer (512) */
  int32_t inter;     /* SwiGLU width of every expert (640) */
  int32_t top_k;     /* routed experts per token (10) */
  int32_t n_shared;  /* shared experts (0 or 1) */
  /* Routing groups G (0 means 1): one (D_g, U_g) pair per group of
   * n_experts / G experts (agentspulse tutorial, section "latent MoE
   * architecture": a layer holds eight such pairs, a label on each expert
   * names its pair; Hugging Face card, "Architecture": the down projection
   * is done per routing group). Reading: expert e belongs to group
   * e / (n_experts / G) (any labelling is this one after renumbering the
   * experts); every token is projected by every D_g; expert e's logit and
   * output use its group's latent h_g = x D_g^T; the shared expert belongs
   * to group 0; out = sum_g z_g U_g^T, z_g the weighted outputs of the
   * token's experts in group g. */
  int32_t n_groups;
} moe_latent_dims;

typedef struct moe_fp4_matrix {
  const uint8_t *codes;  /* [count][N][K/2] (E1M1: [count][N][K/32][12]), 16-byte aligned */
  const uint8_t *scales; /* [count][N][K/16], 16-byte aligned */
  const float *gscale;   /* [count] */
  int32_t bits;          /* element format: 0 or 4 = e2m1, 3 = E1M1 (gate and up only) */
} moe_fp4_matrix;

/* gate and up have one format (bits), the routed and shared sets of a
 * layer the same one, and down is e2m1; else MOE_LATENT_EUNSUPPORTED. E1M1
 * gate/up need latent a multiple of 64. */
typedef struct moe_fp4_experts {
  moe_fp4_matrix gate; /* N = inter,  K = latent */
  moe_fp4_matrix up;   /* N = inter,  K = latent */
  moe_fp4_matrix down; /* N = latent, K = inter  */
  int32_t count;       /* n_experts for the routed set, n_shared for the shared one */
} moe_fp4_experts;

/* Packed copies of a layer's weights for one path (NULL members: not given). */
typedef struct moe_packed_weights {
  const moe_fp4_experts *experts; /* routed experts (count n_experts) */
  const moe_fp4_experts *shared;  /* shared expert (count n_shared); with experts */
  const void *D;                  /* bf16 [latent][hidden] */
  const void *U;                  /* bf16 [hidden][latent] */
  const void *R;                  /* bf16 router.w [n_experts][latent] */
  /* decode path only, optional: the router folded onto the residual width
   * (moe_router_fold). Given, the decode path computes the logits from x in
   * the same launch as h = x D^T and does not read R. */
  const void *RD;
} moe_packed_weights;

/* Packing layouts (moe_fp4_pack, moe_bf16_pack). */
#define MOE_LATENT_PACK_GROUPED 1
#define MOE_LATENT_PACK_DECODE 2

typedef struct moe_router {
  const uint16_t *w; /* bf16 [n_experts][latent], 16-byte aligned */
  const float *bias; /* fp32 [n_experts], or NULL for no bias */
} moe_router;

/* Optional copies of the routing, written when the pointer is non-NULL
 * (device memory). Pair p = t * top_k + j is the j-th choice of token t. */
typedef struct moe_route_debug {
  int32_t *topk_idx; /* [T][top_k], descending logit order */
  float *topk_w;     /* [T][top_k], renormalised weights */
  int32_t *counts;   /* [n_experts] pairs routed to each expert */
  int32_t *offsets;  /* [n_experts + 1] exclusive prefix sum of counts */
  int32_t *perm;     /* [T * top_k] pairs grouped by expert, ascending p within one */
  float *logits;     /* [T][n_experts] router logits (fp32) */
} moe_route_debug;

/* Execution path: the grouped-GEMM pipeline (any T) or the weight-streaming
 * decode kernels (T <= MOE_LATENT_DECODE_MAX_T; hidden and latent multiples
 * of 256 with latent <= 1792, inter a multiple of 128 up to 640, and with
 * routing groups n_experts / G a multiple of 16). AUTO picks the decode
 * kernels whenever T and the dims allow it; DECODE with other sizes returns
 * MOE_LATENT_EUNSUPPORTED. The decode path sums the expert outputs of a
 * token in 64-bit fixed point (units of 2^-32), exact for |z| < 2^31 per
 * latent element; a layer whose combined expert output reaches that
 * magnitude needs the grouped path. With one routing group its gate/up
 * products run in fp16 when every value of bf16(h) converts to fp16
 * exactly (checked per call), else in bf16: the dequantised weights are
 * exact in both, so the products are the same and only the order of the
 * fp32 sums differs between the two. */
#define MOE_LATENT_PATH_AUTO 0
#define MOE_LATENT_PATH_GROUPED 1
#define MOE_LATENT_PATH_DECODE 2
#define MOE_LATENT_DECODE_MAX_T 8

/* Stages of one call, for optional timing (moe_latent_opts.stage_events).
 * The decode path runs four kernels and reports them as DPROJ (D, and with
 * folded router weights the router logits too), ROUTER (the router logits
 * when they are not folded), GATEUP (which also takes the top-k), DOWN
 * (which also combines) and UPROJ. */
#define MOE_LATENT_STAGE_NORM 0     /* RMSNorm of the residual block */
#define MOE_LATENT_STAGE_DPROJ 1    /* h = x D^T */
#define MOE_LATENT_STAGE_ROUTER 2   /* logits = h R^T + b */
#define MOE_LATENT_STAGE_TOPK 3     /* top-k + renormalised weights */
#define MOE_LATENT_STAGE_ROUTE 4    /* histogram, prefix sums, permutation */
#define MOE_LATENT_STAGE_GATEUP 5   /* gate/up GEMMs + SiLU*mul */
#define MOE_LATENT_STAGE_DOWN 6     /* down GEMMs */
#define MOE_LATENT_STAGE_COMBINE 7  /* weighted combine */
#define MOE_LATENT_STAGE_UPROJ 8    /* out = z U^T (+ residual) */
#define MOE_LATENT_N_STAGES 9

typedef struct moe_latent_opts {
  int32_t path;             /* MOE_LATENT_PATH_* */
  int32_t residual;         /* 1: out = x + MoE(rmsnorm(x) * norm_weight) */
  const float *norm_weight; /* fp32 [hidden], required when residual = 1 */
  float norm_eps;           /* RMSNorm epsilon (e.g. 1e-6) */
  /* NULL, or 2 * MOE_LATENT_N_STAGES hipEvent_t created by the caller:
   * entries 2s and 2s+1 (when non-NULL) are recorded on `stream` just
   * before and just after stage s's kernels. Stages a path does not run
   * leave their events untouched. */
  void *const *stage_events;
  /* NULL, or grouped-packed copies of the same weights: the grouped path
   * reads each member given instead of the plain argument (experts and,
   * with n_shared = 1, shared come together; each of D, U, R on its own).
   * Needs latent and inter multiples of 64 for experts, U and R, hidden for
   * D, n_experts % 32 == 0 for R (else MOE_LATENT_EUNSUPPORTED). */
  const moe_packed_weights *grouped_packed;
  /* NULL, or decode-packed copies: all of experts, shared (n_shared = 1),
   * D, U and R or RD (or both), read by the decode path instead of the
   * plain arguments. Needs n_experts % 16 == 0 (the decode path's dims
   * rules give the rest). Neither path reads the other's copies. */
  const moe_packed_weights *decode_packed;
} moe_latent_opts;

/* Device bytes of scratch one call needs for `T` tokens (the maximum over
 * paths, so any path runs with it). Returns 0 for invalid dims or T <= 0. */
size_t moe_latent_workspace_bytes(const moe_latent_dims *dims, int64_t T);

/* The layer forward for T tokens: out = MoE(x). Enqueues every kernel on
 * `stream` (a hipStream_t; NULL = the null stream) and returns without
 * synchronising. T = 0 returns 0 and enqueues nothing once dims and opts
 * are valid (the buffers may then be NULL). `shared` may be NULL
 * only when dims->n_shared = 0. `out` must not overlap `x`. `workspace` is
 * device memory of at least moe_latent_workspace_bytes(dims, T) bytes,
 * 256-byte aligned; its contents need not be initialised. `debug` may be
 * NULL. */
int moe_latent_forward(const moe_latent_dims *dims, int64_t T, const void *x, const void *D,
                       const void *U, const moe_router *router,
                       const moe_fp4_experts *experts, const moe_fp4_experts *shared,
                       void *out, void *workspace, size_t workspace_bytes,
                       moe_route_debug *debug, void *stream);

/* As moe_latent_forward, with options (NULL = defaults: AUTO path, no
 * residual). D, U, router->w, experts and shared may be NULL when the path
 * that runs (decided from opts->path, T and dims before any pointer is
 * checked) has packed copies of them in opts: a decode-packed set stands in
 * for all of them on the decode path, and each member of a grouped-packed
 * set for its plain argument on the grouped path. router->bias is always
 * read from `router`. With opts->residual = 1 this is the residual block
 * out = x + MoE(rmsnorm(x) * norm_weight): the RMSNorm runs in fp32 and its
 * result is rounded to bf16 before D; the residual add is fp32, then rounded. */
int moe_latent_forward_ex(const moe_latent_dims *dims, int64_t T, const void *x, const void *D,
                          const void *U, const moe_router *router,
                          const moe_fp4_experts *experts, const moe_fp4_experts *shared,
                          void *out, void *workspace, size_t workspace_bytes,
                          moe_route_debug *debug, const moe_latent_opts *opts, void *stream);

/* Largest scratch (bytes) the allocation-free entry point serves: every
 * call whose moe_latent_workspace_bytes() is at most this (any decode-path
 * call at the 145B and 120B shapes, T <= 8; grouped-path calls up to a few
 * hundred tokens at those shapes). */
#define MOE_LATENT_NOALLOC_MAX_BYTES ((size_t)32 << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): as
 * moe_latent_forward_ex, without the workspace arguments. The scratch is a
 * static device array of MOE_LATENT_NOALLOC_MAX_BYTES inside the library,
 * one per device, held from the library's first use on that device until
 * the process ends; the call itself allocates and frees nothing. The array
 * used is the one of the calling thread's current device, which must be
 * the device `stream` belongs to (as for any launch). Every call on one
 * device shares that device's array and leaves its contents behind (the
 * kernels need no initialised scratch). Calls enqueued one after another on
 * one stream are ordered by it; calls that can overlap on one GPU (several
 * streams, or several host threads with their own streams) race on the
 * array unless the caller serialises them. Returns MOE_LATENT_EWORKSPACE
 * (before any HIP call) when moe_latent_workspace_bytes(dims, T) exceeds
 * MOE_LATENT_NOALLOC_MAX_BYTES, MOE_LATENT_EHIP if the array's address
 * cannot be obtained; all other arguments and errors as
 * moe_latent_forward_ex. */
int moe_latent_forward_noalloc(const moe_latent_dims *dims, int64_t T, const void *x,
                               const void *D, const void *U, const moe_router *router,
                               const moe_fp4_experts *experts, const moe_fp4_experts *shared,
                               void *out, moe_route_debug *debug, const moe_latent_opts *opts,
                               void *stream);

/* Human-readable description of the last non-zero return on this thread
 * ("" if none). The pointer stays valid until the next call on the thread. */
const char *moe_latent_last_error(void);

/* MOE_LATENT_ABI_VERSION of the library. */
int moe_latent_version(void);

/* Writes `layout` (MOE_LATENT_PACK_GROUPED or _DECODE, see "Layouts") of
 * the fp4 matrix set `src` ([count][N][K] codes and scales in the format
 * src->bits names; gscale is not read) to dst_codes (as many bytes as the
 * source codes: count*N*K/2, or count*N*K*3/8 for E1M1) and dst_scales
 * (count*N*K/16 bytes), device memory, 16-byte aligned, overlapping neither
 * the source nor each other. The packed set keeps the source's bits. Enqueued on `stream`; a one-time step when weights are loaded.
 * Returns MOE_LATENT_EUNSUPPORTED when N, K do not fit the layout (grouped:
 * N % 32, K % 64; decode: N % 16, K % 128), EINVAL for an unknown layout,
 * NULL, misaligned or overlapping buffers. count = 0 enqueues nothing. */
int moe_fp4_pack(const moe_fp4_matrix *src, int32_t count, int32_t N, int32_t K, int32_t layout,
                 uint8_t *dst_codes, uint8_t *dst_scales, void *stream);

/* Writes `layout` of the bf16 matrix `src` [N][K] to `dst` (N*K*2 bytes),
 * device memory, 16-byte aligned, not overlapping src. Enqueued on `stream`.
 * MOE_LATENT_EUNSUPPORTED when N, K do not fit the layout (grouped: N % 32,
 * K % 64; decode: N % 16, K % 32); EINVAL for an unknown layout, NULL,
 * misaligned or overlapping buffers. */
int moe_bf16_pack(const void *src, int32_t N, int32_t K, int32_t layout, void *dst, void *stream);

/* The router folded onto the residual width, for the decode path: since
 * l = h R^T + b with h = x D^T (the layer recipe above), l = x W^T + b with
 * W = R D, [n_experts][hidden] (with routing groups, row e of W is
 * R_e D_{g(e)}). W is accumulated in fp64 and stored as two
 * bf16 matrices, hi = bf16(W) and lo = bf16(W - hi) (together about 16
 * significant bits, as the latent vector's hi + lo halves the unfolded
 * router reads), each in the decode-packed bf16 layout, hi first: dst holds
 * 2 * n_experts * hidden bf16 (device memory, 16-byte aligned, overlapping
 * neither D nor R). D and R are the plain layouts (bf16 [latent][hidden],
 * [n_experts][latent]). A one-time step when weights are loaded, enqueued
 * on `stream`. The decode path reads dst through moe_packed_weights.RD; its
 * logits then agree with the unfolded router's to rounding (not bit for
 * bit). MOE_LATENT_EUNSUPPORTED unless n_experts % 16 == 0 and
 * hidden % 32 == 0; EINVAL for NULL, misaligned or overlapping buffers. */
int moe_router_fold(const moe_latent_dims *dims, const void *D, const void *R, void *dst,
                    void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_LATENT_H */
