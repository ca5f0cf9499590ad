/*
 * pisa.h -- C ABI of the MI355X (gfx950) PISA piecewise sparse attention
 * forward pass.
 *
 * The method (arXiv 2602.01077; gist.science technical summary, section 2
 * "Methodology", subsections "Core Algorithm", "Covariance-Aware Routing" and
 * "Hardware Implementation"; the authors' README, "Kernel variants" and
 * "Attention sink for MMDiT"): per (batch, head), keys and queries are cut into
 * blocks of `block` tokens. Each query block i attends exactly to the top-k key
 * blocks S_i chosen from pooled statistics; every other block j (the set U_i)
 * enters the same softmax numerator and denominator through its zeroth-order
 * Taylor term at the key centroid, and the hybrid variant adds one global
 * first-order correction built from the mean first-order matrix H̄:
 *
 *   o_t = N_t / D_t,  α_tj = exp(s q_t·k̄_j),
 *   N_t = Σ_{j∈S_i} Σ_n e^{s q_t·k_n} v_n + Σ_{j∈U_i} α_tj ΣV_j
 *         + [hybrid] (Σ_{j∈U_i} α_tj) · s · q_t H̄,
 *   D_t = Σ_{j∈S_i} Σ_n e^{s q_t·k_n} + Σ_{j∈U_i} n_j α_tj.
 *
 * Conventions for every entry point:
 *  - Tensors q, k, v, o are DEVICE pointers to contiguous arrays of the I/O
 *    dtype, [B, H, L, D] or [B, L, H, D] as shape->layout says, owned by the
 *    caller, 16-byte aligned.
 *  - n = ceil(L / block) blocks per (batch, head); the last one holds
 *    n_last = L - (n-1)*block tokens.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and runs asynchronously; the caller keeps every buffer alive until the
 *    stream has passed the call. No entry point synchronises the device or
 *    allocates device memory: scratch space is the caller's workspace, or for
 *    pisa_attn_fwd_noalloc a fixed array that is part of the library's code
 *    object on each device.
 *  - Arguments are validated before anything is enqueued. A bad argument
 *    returns PISA_EINVAL and enqueues nothing; a combination the library does
 *    not build returns PISA_ENOTSUP; a launch failure reported by the HIP
 *    runtime returns PISA_EHIP. No call aborts the process or throws.
 *  - The state the library keeps: a per-host-thread copy of the text of the
 *    last HIP error (pisa_last_hip_error), and for pisa_attn_fwd_noalloc one
 *    fixed scratch array per device. Calls from several host threads at once
 *    are safe as long as they use different workspaces (and, for
 *    pisa_attn_fwd_noalloc, different devices).
 */
#ifndef PISA_H_
#define PISA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PISA_OK = 0,
  PISA_EINVAL = 1,  /* invalid argument; nothing enqueued */
  PISA_ENOTSUP = 2, /* valid but not built (e.g. an unsupported head_dim) */
  PISA_EHIP = 3,    /* the HIP runtime reported a launch error */
  PISA_ETOOBIG = 4  /* pisa_attn_fwd_noalloc: the problem needs more than its fixed scratch */
} pisa_status_t;

typedef enum { PISA_F32 = 0, PISA_BF16 = 1 } pisa_dtype_t;

/* Memory layout of q, k, v and o, all contiguous:
 * PISA_LAYOUT_BHLD [B,H,L,D], the layout of the README's functions;
 * PISA_LAYOUT_BLHD [B,L,H,D], the layout attention processors of DiT models
 * hold q, k, v in before their head transpose (README, the diffusers
 * processor integration), read in place without a transposed copy. Block
 * statistics, selections and workspace copies do not depend on it. */
#define PISA_LAYOUT_BHLD 0
#define PISA_LAYOUT_BLHD 1

/* Problem shape. Supported: D in {64, 128}, block in {64, 128}, L >= 1,
 * B*H >= 1, n = ceil(L / block) <= 8192, dtype PISA_F32 or PISA_BF16 (the I/O
 * dtype; see pisa_stats_t for the precision of each statistic; the fused
 * pass accumulates in fp32), layout PISA_LAYOUT_BHLD or PISA_LAYOUT_BLHD (a
 * zero-initialised shape is BHLD). */
typedef struct {
  int32_t B, H, L, D, block;
  int32_t dtype;  /* pisa_dtype_t */
  int32_t layout; /* PISA_LAYOUT_* */
} pisa_shape_t;

#define PISA_SINK_NONE INT32_MIN /* sink_idx values: PISA_SINK_NONE, 0, -1 */

/* Block statistics (gist summary, "Hardware Implementation", pre-computation
 * step; symbols of "Core Algorithm"). All pointers are caller-owned device
 * buffers of the sizes given; n = ceil(L / block).
 *   qbar  [B,H,n,D] fp64  mean of the query rows of block i
 *   kbar  [B,H,n,D] fp64  key centroid k̄_j (mean of the block's keys)
 *   vsum  [B,H,n,D] fp64  ΣV_j, the sum (not mean) of the block's values
 *   hbar  [B,H,D,D] fp64  H̄[d][e] = (1/n) Σ_j Σ_n (k_n - k̄_j)[d] v_n[e]
 *   mnorm [B,H,n]   fp64  M_j = ||H_j - H̄|| in the norm mnorm_ord names
 *                         (below); may be NULL unless the covariance-aware
 *                         routing of pisa_select is used
 *   ws / ws_bytes         workspace of at least pisa_workspace_bytes(shape)
 *                         bytes, 256-byte aligned (see below).
 * Precision: q̄, k̄ and ΣV are fp64 sums of the inputs (exact for bf16),
 * divided in fp64. H̄ is the mean of per-block H_j formed in fp32 on the
 * matrix cores: the products k[d]·v[e] are exact for bf16 inputs, each run of
 * consecutive blocks (up to 1024 tokens) is summed in one fp32 accumulator,
 * from which k̄_j[d]·ΣV_j[e] (rounded to fp32) is subtracted as block j ends,
 * and the runs are summed in fp64. The Frobenius M_j takes the block's fp32
 * sum of products, subtracts k̄_j[d]·ΣV_j[e] and H̄ in fp64, and sums the
 * squares in fp64; the spectral M_j sums the block's products in fp64.
 * The workspace: pisa_block_stats writes there the copies of K, V, k̄, ΣV and
 * H̄ in the I/O dtype, laid out in the operand order of the fused kernel, and
 * the largest key norms; for rows of more than 1280 blocks pisa_select
 * stages its routing scores there (shorter rows are scored and selected on
 * chip);
 * pisa_attn_fwd reads the copies and resets and uses two counters there (the
 * tiles left to its running-maximum kernel, and the arrival count that keeps
 * its workgroups in step). A workspace therefore serves one call at a time:
 * calls that share one must be ordered, e.g. on one stream. */
typedef struct {
  double *qbar, *kbar, *vsum, *hbar, *mnorm;
  void *ws;
  size_t ws_bytes;
  int32_t mnorm_ord; /* PISA_NORM_FRO (0, a zeroed struct) or PISA_NORM_SPECTRAL */
} pisa_stats_t;

/* The norm of M_j = ||H_j - H̄||: Frobenius (the square root of the sum of
 * squares, as the skill page's scoring code takes it), or spectral, the
 * largest singular value (the 2-norm the gist's "Covariance-Aware Routing"
 * writes). The spectral norm is found by a fixed number of fp64 steps per
 * block, whatever the gap between the largest singular values: the Gram
 * matrix (H_j - H̄)ᵀ(H_j - H̄) is formed in fp64 from the block's keys and
 * values, reduced to tridiagonal form by Householder reflections and its
 * largest eigenvalue found by Sturm-count bisection. It costs one workgroup
 * of about D³ fp64 work per block, so it suits image-sized sequences (the
 * pages apply covariance-aware routing to images). Any other value of
 * mnorm_ord: PISA_EINVAL. */
#define PISA_NORM_FRO 0
#define PISA_NORM_SPECTRAL 2

/* Bytes of workspace the stats / select / forward calls need for `shape`
 * (0 if the shape is invalid). */
size_t pisa_workspace_bytes(const pisa_shape_t *shape);

/* Step 1: block statistics. Reads q, k, v once; writes qbar, kbar, vsum,
 * hbar (and mnorm when non-NULL) plus the workspace copies. */
pisa_status_t pisa_block_stats(const pisa_shape_t *shape, const void *q, const void *k,
                               const void *v, const pisa_stats_t *st, void *stream);

/* Step 2: per-query-block top-k routing (gist summary, "Covariance-Aware
 * Routing"; README, "Attention sink for MMDiT"). Score of key block j for
 * query block i: S_ij = scale * q̄_i·k̄_j + cov_weight * M_j (fp64), and
 * +infinity for the sink block (sink_idx 0: block 0; -1: block n-1;
 * PISA_SINK_NONE: none). The topk largest scores win; equal scores go to the
 * lower block index. idx [B,H,n,topk] int32 (device, caller-owned) receives
 * each query block's selection in ascending order.
 * Requires: 1 <= topk <= n; cov_weight >= 0 and finite; st->mnorm non-NULL
 * (computed by pisa_block_stats) when cov_weight > 0; the workspace of
 * pisa_block_stats (the routing scores of rows longer than 1280 blocks are
 * staged there). */
pisa_status_t pisa_select(const pisa_shape_t *shape, const pisa_stats_t *st, double scale,
                          double cov_weight, int32_t topk, int32_t sink_idx, int32_t *idx,
                          void *stream);

/* Step 3: fused exact + Taylor online-softmax pass (gist summary, "Core
 * Algorithm" N_t equation and "Hardware Implementation" phases 1-3).
 * first_order = 1: hybrid variant (zeroth order plus global first-order
 * correction, the paper version); 0: zeroth-order-only variant (README,
 * "Kernel variants"); 2: per-block first-order variant, every unselected
 * block with its own first-order term alpha_tj * scale * q_t H_j (the
 * distinct per-block terms that the gist's "Core Algorithm" replaces by the
 * global mean H-bar; the first-order variant of the atlas summary's results),
 * evaluated over the block's keys in one sweep over all key blocks, so it
 * costs about as much as dense attention. Any other value: PISA_EINVAL.
 * idx [B,H,n,topk] int32, each row ascending without
 * repeats, entries in [0, n) (any selection is accepted, e.g. one computed
 * elsewhere; entries outside [0, n) are clamped into it, so they cannot read
 * out of bounds). The call takes no k and v: keys, values, k̄, ΣV and H̄ are
 * read from the copies that the last pisa_block_stats on st->ws wrote, so the
 * result is attention over the k and v of that call (the library cannot
 * check that they belong to this q). o, shaped like q, receives the output in
 * the I/O dtype (round to nearest even). */
pisa_status_t pisa_attn_fwd(const pisa_shape_t *shape, const void *q, const pisa_stats_t *st,
                            int32_t first_order, const int32_t *idx, int32_t topk, double scale,
                            void *o, void *stream);

/* pisa_attn_fwd that also writes, for every row t, lse[t] = ln D_t: the
 * natural log of the row's denominator D_t (the gist's "Core Algorithm", the
 * same for all three variants up to rounding), taken over the unshifted
 * exponentials e^{scale q_t·k}. lse is a caller-owned device buffer of
 * [B,H,L] fp32 (4-byte aligned, in this order whatever shape->layout is).
 * It is what pisa_attn_bwd can take instead of recomputing the denominators.
 * Errors as for pisa_attn_fwd, and PISA_EINVAL for a NULL or misaligned lse. */
pisa_status_t pisa_attn_fwd_lse(const pisa_shape_t *shape, const void *q, const pisa_stats_t *st,
                                int32_t first_order, const int32_t *idx, int32_t topk, double scale,
                                void *o, float *lse, void *stream);

/* Backward pass of the zeroth-order-only variant (first_order = 0), the form
 * the README's "Kernel variants" names as the one that supports training.
 * With the selection idx held fixed, the gradients of L = Σ o∘dout follow from
 * the N_t / D_t of pisa_attn_fwd by the chain rule; the block centroid k̄_j
 * and the value sum ΣV_j of an unselected block pass their gradients on to
 * every token of block j (dk_n gets dk̄_j / n_j, dv_n gets dΣV_j).
 *   q, k, v   the forward's inputs (one tensor each; shape->layout as there)
 *   st        the forward's statistics: st->kbar and st->vsum are read (the
 *             workspace copies are not)
 *   idx, topk the forward's selection, as for pisa_attn_fwd
 *   o         the forward's output (o_t enters through Δ_t = dout_t·o_t)
 *   lse       NULL, or the [B,H,L] fp32 ln D_t that pisa_attn_fwd_lse wrote
 *             for this forward call; with NULL the backward recomputes the
 *             denominators in one more sweep over every row's keys
 *   dout      the gradient of the loss with respect to o
 *   dq, dk, dv receive the gradients, shaped and typed like q, k, v
 *   ws        at least pisa_bwd_workspace_bytes(shape) bytes, 256-aligned:
 *             the selection as a bitmap, each row's log-sum of weights and
 *             Δ_t, the fp32 gradients of k̄ and ΣV (for short sequences
 *             also their partial sums over ranges of query blocks), and a
 *             counter, reset by each call, that keeps the dq workgroups in
 *             step; a workspace serves one call at a time (order calls that
 *             share one, e.g. on one stream)
 * Products run on the matrix cores with fp32 accumulation; the weights and
 * their gradients are rounded to the I/O dtype as operands. Deterministic.
 * Errors as for pisa_attn_fwd. */
size_t pisa_bwd_workspace_bytes(const pisa_shape_t *shape);
pisa_status_t pisa_attn_bwd(const pisa_shape_t *shape, const void *q, const void *k, const void *v,
                            const pisa_stats_t *st, const int32_t *idx, int32_t topk, double scale,
                            const void *o, const float *lse, const void *dout, void *dq, void *dk,
                            void *dv, void *ws, size_t ws_bytes, void *stream);

/* pisa_block_stats followed by pisa_attn_fwd in one call that allocates
 * nothing and takes no workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Every intermediate (the operand copies of K and V, the
 * block statistics, the partial sums and the counters) lives in one fixed
 * array of PISA_NOALLOC_SCRATCH_BYTES per device, which the library holds
 * from its first call on that device until the process ends; the caller
 * passes only q, k, v, the selection and the output, with the meanings and
 * layouts of pisa_block_stats and pisa_attn_fwd (one tensor per sequence,
 * no covariance norm). The output equals that of pisa_block_stats +
 * pisa_attn_fwd on the same arguments bit for bit.
 * Returns PISA_ETOOBIG, enqueueing nothing, when the shape needs more
 * scratch than that (about B*H*L*D*2*esz bytes of operand copies plus the
 * statistics: FLUX-sized calls fit, a Wan-sized call does not). Every call on
 * one device shares its array, and each call resets what must start at zero:
 * calls that overlap on one device (on different streams, or from several
 * host threads) race and give undefined results; order them on one stream. */
#define PISA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
pisa_status_t pisa_attn_fwd_noalloc(const pisa_shape_t *shape, const void *q, const void *k,
                                    const void *v, int32_t first_order, const int32_t *idx,
                                    int32_t topk, double scale, void *o, void *stream);

/* Same-device dense baseline: o = softmax(scale * Q Kᵀ) V per (batch, head)
 * (the skill page's compute_exact_attention, used as the definition of dense
 * attention), computed by the same tile loop as pisa_attn_fwd's exact phase
 * over every key block. ws: at least dense_workspace_bytes(shape) bytes,
 * 256-byte aligned (operand-ordered K and V copies). */
size_t dense_workspace_bytes(const pisa_shape_t *shape);
pisa_status_t dense_attn_fwd(const pisa_shape_t *shape, const void *q, const void *k,
                             const void *v, double scale, void *o, void *ws, size_t ws_bytes,
                             void *stream);

/* Joint attention over a sequence held in two tensors (README, "Attention
 * sink for MMDiT": MMDiT blocks attend over the text and image token streams
 * as one sequence, with the text block as the sink: sink_idx 0 when the text
 * comes first, -1 when it comes last). Tokens [0, L0) of the sequence are in
 * the q, k, v (and o) arguments, which then hold L0 tokens; tokens [L0, L)
 * are in q1, k1, v1 (and o1), which hold L - L0 tokens. Both parts have the
 * shape's layout and dtype; shape->L is the joint length. No concatenated
 * copy is made: the kernels address each token in its own tensor. The
 * segment boundary need not fall on a block boundary.
 * Requires 1 <= L0 <= L; when L0 < L, the second-segment pointers the call
 * reads or writes are non-NULL and 16-byte aligned (L0 == L: they are
 * ignored). Otherwise PISA_EINVAL. A NULL pisa_segments_t is the
 * one-tensor case. */
typedef struct {
  int32_t L0;
  const void *q1, *k1, *v1;
  void *o1;
} pisa_segments_t;

/* pisa_block_stats on a two-part sequence (reads seg->q1, k1, v1). */
pisa_status_t pisa_block_stats_seg(const pisa_shape_t *shape, const void *q, const void *k,
                                   const void *v, const pisa_segments_t *seg,
                                   const pisa_stats_t *st, void *stream);

/* pisa_attn_fwd on a two-part sequence (reads seg->q1, writes seg->o1). st
 * comes from pisa_block_stats_seg with the same segments; pisa_select is
 * unchanged. */
pisa_status_t pisa_attn_fwd_seg(const pisa_shape_t *shape, const void *q, const pisa_stats_t *st,
                                int32_t first_order, const int32_t *idx, int32_t topk,
                                double scale, void *o, const pisa_segments_t *seg, void *stream);

/* dense_attn_fwd on a two-part sequence (reads seg->q1, k1, v1, writes o1). */
pisa_status_t dense_attn_fwd_seg(const pisa_shape_t *shape, const void *q, const void *k,
                                 const void *v, const pisa_segments_t *seg, double scale, void *o,
                                 void *ws, size_t ws_bytes, void *stream);

/* Human-readable text of a status code (static storage). */
const char *pisa_status_string(pisa_status_t status);

/* Text of the last HIP error seen by a call on this host thread ("" if none). */
const char *pisa_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* PISA_H_ */
