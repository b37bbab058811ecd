/*
 * pisa.h - C ABI of libpisa, the gfx950 (MI355X) forward path of PISA
 * piecewise sparse attention.
 *
 * Method: "PISA: Piecewise Sparse Attention Is Wiser for Efficient Diffusion
 * Transformers" (arXiv 2602.01077), §3.2 Eqs. 3-6, §3.3 Eqs. 9-10, §3.4
 * Algorithm 1; the optional second-order mass term and its gate follow the
 * "Piecewise-Taylor-Attention" README ("Blog post" section and changelog).
 *
 * The operator is split along the paper's own phases (Algorithm 1, "Prepare
 * Phase" steps 1-2, then the fused kernel's Phases 1-3):
 *
 *   pisa_block_stats  - per-KV-block statistics and the global H   (step 1)
 *   pisa_route_topk   - pooled-score routing, top-k per query block (step 2)
 *   pisa_attn_fwd     - exact + virtual-token + global first order (Phases 1-3)
 *
 * Conventions shared by all entry points
 * --------------------------------------
 * - Tensors q, k, v, o are [batch, heads, seq_len, head_dim] row-major and
 *   contiguous, in the dtype named by pisa_shape_t.dtype (PISA_BF16: bf16
 *   storage; PISA_F32: fp32). N = ceil(seq_len / block_size) blocks; block j
 *   holds rows [64 j, min(64 j + 64, seq_len)); the last block may be partial.
 * - Every pointer argument is a DEVICE pointer (HBM), except the shape and
 *   parameter structs, which are host pointers read during the call.
 * - All work is enqueued asynchronously on `stream` (a hipStream_t; NULL is
 *   the null stream). No call synchronises, allocates or frees memory; the
 *   caller owns every buffer, sized with the helpers below.
 * - Every argument is validated on the host before any HIP call; a failing
 *   check returns a status and enqueues nothing. A launch failure returns
 *   PISA_ERR_HIP. Faults inside kernels surface at the caller's next
 *   synchronisation. Device data are not validated on the host; routing
 *   table entries outside [0, N) are ignored by the kernels (see
 *   pisa_attn_fwd).
 * - Results are deterministic: no floating-point atomics, fixed reduction
 *   orders, identical bits for identical inputs and launch shapes.
 * - Softmax scale s = shape.scale, or 1/sqrt(head_dim) when scale <= 0; it
 *   multiplies every logit (exact, virtual and routing), and the Taylor
 *   terms use q' = s q (Appendix C of the paper puts 1/sqrt(d) in alpha).
 */
#ifndef PISA_H_
#define PISA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PISA_ABI_VERSION 15

typedef enum {
    PISA_OK = 0,
    PISA_ERR_NULL = 1,        /* a required pointer is NULL                         */
    PISA_ERR_SHAPE = 2,       /* batch/heads/seq_len/head_dim out of range           */
    PISA_ERR_DTYPE = 3,       /* unknown dtype                                      */
    PISA_ERR_PARAM = 4,       /* topk, band, flags or scale out of range            */
    PISA_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned                   */
    PISA_ERR_UNSUPPORTED = 6, /* valid request this build does not implement        */
    PISA_ERR_HIP = 7,         /* a HIP launch or runtime call failed                */
    PISA_ERR_WORKSPACE = 8    /* workspace smaller than pisa_stats_workspace_bytes   */
} pisa_status_t;

typedef enum { PISA_F32 = 0, PISA_BF16 = 1 } pisa_dtype_t;

typedef struct {
    int64_t batch;      /* >= 1                                            */
    int64_t heads;      /* >= 1                                            */
    int64_t seq_len;    /* T >= 1, at most 524288 (N <= 8192 blocks)         */
    int64_t head_dim;   /* D, 64 or 128                                     */
    int32_t block_size; /* B; must be 64 (the paper's kernel block, §4.1)   */
    int32_t dtype;      /* pisa_dtype_t of q, k, v, o                       */
    float scale;        /* softmax scale; <= 0 selects 1/sqrt(head_dim)     */
} pisa_shape_t;

typedef struct {
    int32_t topk;         /* routed KV blocks per query block, band excluded, 0..N */
    int32_t band;         /* |i - j| <= band is always exact (>= 0)               */
    int32_t second_order; /* 1: add the gated second-order term w (README)        */
    int32_t first_order;  /* 1: global first order (Eq. 10, Phase 3); 0: off     */
    int32_t phase_mask;   /* 0 = all phases; bit0 exact, bit1 virtual, bit2 first
                             order (measurement only)                            */
    int32_t n_sink;       /* the first n_sink KV blocks are exact for every query
                             block, like the band (README knobs: n_sink_blocks,
                             e.g. an MMDiT text prefix); 0..N                    */
    int32_t cov_bias;     /* 1: covariance-aware routing (Eq. 11): the routing
                             score gains log(M_j + PISA_COV_EPS), M_j = hnorm[j];
                             pisa_block_stats then also computes hnorm        */
} pisa_params_t;

/* eps of the covariance prior log(M_j + eps) (Eq. 11 leaves it unvalued) */
#define PISA_COV_EPS 1e-6

/*
 * Block statistics (Algorithm 1 step 1 and Fig. 4 "Prepare Phase": block
 * means of Q and K, block value sums, the global first-order matrix; §3.2
 * Formulation; Appendix C; README "Blog post" for the key variance and the
 * pooled q^2). All are caller-owned device arrays:
 *   qbar[i]   = (1/n_i) sum_t q_t                      fp64 [B,H,N,D]
 *   q2bar[i]  = (1/n_i) sum_t (s q_t)^2  (elementwise)  fp64 [B,H,N,D]
 *   kbar[j]   = (1/n_j) sum_n k_{j,n}                  fp64 [B,H,N,D]
 *   vsum[j]   = sum_n v_{j,n}               (V-hat)    fp32 [B,H,N,D]
 *   ksig2[j]  = (1/n_j) sum_n (k_{j,n} - kbar_j)^2     fp64 [B,H,N,D]
 *   hsum      = sum_j sum_n (k_{j,n} - kbar_j)^T v_{j,n}
 *                                            (D x D)   fp32 [B,H,D,D]
 *               (row index: key dim, column index: value dim)
 *   hnorm[j]  = || H_j - Hbar ||_F, H_j = sum_n (k_{j,n} - kbar_j)^T v_{j,n},
 *               Hbar = (1/N) sum_j H_j (the block heterogeneity M_j of
 *               Eq. 11 and Appendix D, with the Frobenius norm the README's
 *               router uses)                            fp64 [B,H,N]
 * n_i, n_j are the rows present in the block (the last one may be partial).
 * qbar, kbar, q2bar and ksig2 are fp64 so that routing decisions (a top-k, a
 * gate) can match a float64 evaluation; q2bar and ksig2 may be NULL unless
 * params.second_order; hnorm may be NULL unless params.cov_bias (it is
 * computed from H_j and Hbar in fp64 from the exact inputs, in two more passes
 * over k and v). pisa_block_stats computes them from q, k, v; a caller
 * may also fill them by any other means and hand them to
 * pisa_prepare_operands.
 */
typedef struct {
    double *qbar;
    double *q2bar;
    double *kbar;
    float *vsum;
    double *ksig2;
    float *hsum;
    double *hnorm;
} pisa_stats_t;

/*
 * The operand buffer: one caller-owned device allocation of
 * pisa_operands_bytes(shape) bytes holding the kernels' own arrangements of
 * the statistics (and of K), which the routing and attention kernels read
 * with contiguous matrix-core operand loads. Its contents are produced by
 * pisa_block_stats (fused with the statistics) or by pisa_prepare_operands
 * (from statistics of any source); they are opaque to callers. Its size
 * depends on the shape only. For diagnostics, pisa_operands_offsets reports
 * where each arrangement starts:
 *   PISA_OPERAND_KBAR_C   kbar rounded to fp32, then to the input dtype [B,H,N,D]
 *   PISA_OPERAND_VBAR_C   (vsum / n_j, in fp64 from the fp32 vsum) rounded to
 *                         fp32, then to the input dtype                 [B,H,N,D]
 *   PISA_OPERAND_KBAR_R   kbar split into bf16 hi = rn(kbar), lo = rn(kbar - hi),
 *                         router order: key j = 16 c + n, dim d = (D/4) g + 8 s + e
 *                         (g < 4, s < D/32, e < 8), part p (hi, lo) at bf16 element
 *                         ((c D/32 + s) 2 + p) 512 + (16 g + n) 8 + e,
 *                         [B,H,ceil(N/16) 16 D 2]; slots of keys past N unspecified
 *   PISA_OPERAND_KSIG2_R  ksig2 the same way (second order only)
 *   PISA_OPERAND_KPACK    bf16 only: K per block j, 32-row half h, chunk c
 *                         (dims 8c..8c+7), row r: element ((h D/8 + c) 32 + r) 8 + e
 *                         = k[64 j + 32 h + r][8 c + e]; 0 past seq_len   [B,H,N,64 D]
 *   PISA_OPERAND_KBPACK   bf16 only: kbar_c rows per group of 64 blocks in
 *                         KPACK's order, 0 past N                    [B,H,ceil(N/64),64 D]
 *   PISA_OPERAND_HPACK    bf16 only: hsum split into bf16 hi + lo, element
 *                         (((dt D/16 + ks) 2 + p) 64 + l) 8 + e = part p of
 *                         hsum[16 ks + 8 (l/32) + e][32 dt + l % 32]     [B,H,2 D D]
 *   PISA_OPERAND_KNORM    fp32 ||kbar_j||_2, rounded up        [B,H,ceil(N/16) 16]
 */
typedef enum {
    PISA_OPERAND_KBAR_C = 0,
    PISA_OPERAND_VBAR_C = 1,
    PISA_OPERAND_KBAR_R = 2,
    PISA_OPERAND_KSIG2_R = 3,
    PISA_OPERAND_KPACK = 4,
    PISA_OPERAND_KBPACK = 5,
    PISA_OPERAND_HPACK = 6,
    PISA_OPERAND_KNORM = 7,
    PISA_OPERAND_COUNT = 8
} pisa_operand_t;

/* ABI version of the library (PISA_ABI_VERSION). */
int pisa_abi_version(void);

/* Human-readable name of a status code (static storage). */
const char *pisa_status_str(pisa_status_t s);

/* N = ceil(seq_len / block_size), or -1 if the shape is invalid. */
int64_t pisa_num_blocks(const pisa_shape_t *shape);

/* Bytes of device workspace pisa_block_stats needs (partial H sums, and with
 * params.cov_bias the fp64 partial sums and Hbar of the prior; the larger of
 * the two, so any params fit), or 0 if the shape is invalid. */
size_t pisa_stats_workspace_bytes(const pisa_shape_t *shape);

/* Bytes of the operand buffer for this shape, or 0 if the shape is invalid. */
size_t pisa_operands_bytes(const pisa_shape_t *shape);

/* Byte offset of each pisa_operand_t arrangement inside the operand buffer
 * (offsets[PISA_OPERAND_COUNT]; an arrangement the dtype does not use gets
 * the offset of the next one and no bytes). Host only, for diagnostics. */
pisa_status_t pisa_operands_offsets(const pisa_shape_t *shape, int64_t *offsets);

/*
 * pisa_block_stats: reads q, k, v once; writes every field of `out` (q2bar
 * and ksig2 only if params->second_order) and fills the operand buffer
 * `operands` (at least pisa_operands_bytes(shape) bytes). `workspace` is
 * caller-owned device memory of at least pisa_stats_workspace_bytes(shape)
 * bytes; its contents on entry are ignored and on return are unspecified.
 * Outputs must not alias inputs.
 */
pisa_status_t pisa_block_stats(const pisa_shape_t *shape, const pisa_params_t *params,
                               const void *q, const void *k, const void *v,
                               const pisa_stats_t *out, void *operands, size_t operands_bytes,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * pisa_block_stats_noalloc: pisa_block_stats for callers that cannot
 * allocate device memory or hand in a workspace (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation). The same
 * kernels and results as pisa_block_stats; the partial H sums go to a static
 * device array of PISA_STATS_SCRATCH_BYTES that the library holds on each GPU
 * it runs on until the process ends (its address is looked up once per
 * device, on the first call there). No allocation happens in the call.
 * Shapes whose scratch need exceeds PISA_STATS_SCRATCH_BYTES (the partial H
 * sums: for head_dim 128, batch * heads > 512; with params.cov_bias the fp64
 * partials of the prior: batch * heads > 128) are rejected with
 * PISA_ERR_WORKSPACE before any HIP call. Every call on one GPU uses that
 * GPU's one array: calls that overlap on one GPU (other streams, other
 * threads) race and must be serialised by the caller. The array needs no
 * clearing: each call writes every partial it reads.
 */
#define PISA_STATS_SCRATCH_BYTES ((size_t)32 << 20)
pisa_status_t pisa_block_stats_noalloc(const pisa_shape_t *shape, const pisa_params_t *params,
                                       const void *q, const void *k, const void *v,
                                       const pisa_stats_t *out, void *operands,
                                       size_t operands_bytes, void *stream);

/*
 * pisa_prepare_operands: fills the operand buffer from statistics of any
 * source (for example ones computed elsewhere, or by a reference
 * implementation): reads stats->kbar, vsum, hsum (and ksig2 if
 * params->second_order) and, for bf16 inputs, k (for PISA_OPERAND_KPACK).
 * For statistics pisa_block_stats wrote, the buffer equals the one
 * pisa_block_stats filled, bit for bit.
 */
pisa_status_t pisa_prepare_operands(const pisa_shape_t *shape, const pisa_params_t *params,
                                    const void *k, const pisa_stats_t *stats, void *operands,
                                    size_t operands_bytes, void *stream);

/*
 * pisa_route_topk (Algorithm 1 step 2 with the pooled score of Eq. 11;
 * README router): for each query block i,
 *   r_ij = s qbar_i . kbar_j + [second_order] min(w_ij, ln B)
 *          + [cov_bias] log(hnorm_j + PISA_COV_EPS),
 *   w_ij = 1/2 q2bar_i . ksig2_j,
 * over the candidates j with |i - j| > band. idx[b,h,i,:] receives the
 * min(topk, #candidates) best j (ties: lower j wins), ascending, then -1.
 * Every decision equals a float64 evaluation of r (scores are computed in
 * fp32 and every block within the fp32 error bound of the cut is re-ranked
 * in fp64).
 * idx: int32 [B,H,N,topk] (may be NULL iff topk == 0).
 * wgate: fp32 [B,H,N,N], required iff second_order: the gated term used by
 *   the virtual-token logits: w_ij where w_ij <= ln B, and 0 where w_ij is
 *   larger (the README's gate, not a clamp), decided as in float64.
 * Reads stats->qbar, kbar (and q2bar, ksig2 if second_order; hnorm if
 * cov_bias) and the operand buffer.
 */
pisa_status_t pisa_route_topk(const pisa_shape_t *shape, const pisa_params_t *params,
                              const pisa_stats_t *stats, const void *operands,
                              size_t operands_bytes, int32_t *idx, float *wgate, void *stream);

/*
 * pisa_attn_fwd (Algorithm 1 Phases 1-3, Eqs. 3-5 and 9-10): for each query
 * row t of block i, with S_i = {|i-j| <= band} U idx[i] and U_i its
 * complement,
 *   o_t = (sum_{j in S_i} sum_n e^{s q.k} v  +  sum_{j in U_i} e^{lam} V-hat_j
 *          + F_t) / (sum_{j in S_i} sum_n e^{s q.k}  +  l_tail_t),
 *   lam_tj = s q_t.kbar_j + [second_order] wgate_ij,
 *   l_tail_t = sum_{j in U_i} n_j e^{lam_tj},
 *   F_t = first_order ? (l_tail_t / T) (s q_t) H : 0.
 * idx rows hold distinct block ids outside the band, then -1 padding (as
 * pisa_route_topk writes them). An entry outside [0, N), at any position, is
 * ignored like -1 (the kernels address no memory from it); a repeated id or
 * one inside the band makes the result unspecified. o: [B,H,T,D] in the input
 * dtype; must not alias q, k, v. bf16 runs compute QK^T and PV with bf16 MFMA (fp32
 * accumulation, P rounded to bf16); fp32 runs compute every product on the
 * fp32 matrix cores (fp32 products and sums; P, kbar and V-hat stay fp32).
 * row_stats: NULL, or a [B,H,T,2] fp32 output (it must not overlap o, q, k,
 * v): for each row t, row_stats[t][0] = lse_t = ln(sum_{j in S_i} sum_n
 * e^{s q.k} + l_tail_t), the natural log of the output's denominator, and
 * row_stats[t][1] = c_t = first_order ? l_tail_t / (T (that denominator)) :
 * 0, the weight of F_t per unit of (s q_t) H after normalisation. They are
 * the per-row quantities pisa_attn_bwd would otherwise recompute (both
 * follow from the same sums as o; a row whose output is NaN gets NaN).
 * Reads the operand buffer (bf16) or stats->vsum, kbar and hsum (fp32).
 */
pisa_status_t pisa_attn_fwd(const pisa_shape_t *shape, const pisa_params_t *params,
                            const void *q, const void *k, const void *v,
                            const pisa_stats_t *stats, const void *operands,
                            size_t operands_bytes, const int32_t *idx,
                            const float *wgate, void *o, float *row_stats, void *stream);

/*
 * pisa_attn_fwd_valu: the same contract as pisa_attn_fwd, computed by a plain
 * fp32 VALU kernel for either dtype (bf16 inputs are widened exactly; P is
 * not rounded, one thread per query row). It is a GPU reference for the
 * matrix-core kernels of pisa_attn_fwd (bf16 and fp32).
 */
pisa_status_t pisa_attn_fwd_valu(const pisa_shape_t *shape, const pisa_params_t *params,
                                 const void *q, const void *k, const void *v,
                                 const pisa_stats_t *stats, const void *operands,
                                 size_t operands_bytes, const int32_t *idx,
                                 const float *wgate, void *o, float *row_stats, void *stream);

/*
 * pisa_attn_fwd_plan (HOST only, no GPU work): which kernel pisa_attn_fwd runs
 * for this shape and these parameters, and the longest item list one wave of
 * the persistent bf16 kernel would build.
 *   kernel      PISA_KERNEL_MFMA_F32 (fp32 inputs), PISA_KERNEL_MFMA_ASM (bf16,
 *               head_dim 128, and a query block's item list fits 512
 *               entries) or PISA_KERNEL_MFMA (bf16 otherwise: head_dim 64,
 *               or lists too long for the persistent kernel);
 *   wave_items  E + G with E = min(N, 2 band + 1 + n_sink) + topk (forced
 *               blocks and routed ids: the exact items) and G = ceil(N / 64)
 *               (the virtual-token groups): one wave of the persistent
 *               kernel lists all of a query block's items.
 * Either output pointer may be NULL. Returns the validation status of shape
 * and params (as pisa_attn_fwd checks them). A band larger than N is taken
 * as N by every entry point.
 */
typedef enum { PISA_KERNEL_VALU = 0, PISA_KERNEL_MFMA_ASM = 1, PISA_KERNEL_MFMA = 2,
               PISA_KERNEL_MFMA_F32 = 3 } pisa_attn_kernel_t;
pisa_status_t pisa_attn_fwd_plan(const pisa_shape_t *shape, const pisa_params_t *params,
                                 int32_t *kernel, int64_t *wave_items);

/*
 * Morton token reorder ("Piecewise-Taylor-Attention" README: the Wan2.1
 * results paragraph, where the 64-token blocks are taken over a Morton
 * (Z-order) tile reordering of the latent grid so that each block is a
 * compact 3D neighbourhood, and the changelog item on the Morton tile reorder
 * with its fused gather kernel). Not part of the operator itself: callers
 * holding token-major activations [B,T,H,D] in raster order use it before and
 * after the three calls above.
 *
 * pisa_z_order (HOST pointers; no GPU work): fills perm[0 .. n) with the
 * visiting order of `prefix` fixed tokens followed by the cells of a grid
 * (grid[0 .. ndim), slowest axis first, raster-numbered after the prefix).
 * A cell's code interleaves the bits of its coordinates: bit b of the axis
 * in slot a (slot 0 = the fastest axis) is code bit ndim*b + a; cells are
 * visited in ascending code (a grid that is not a power of two per axis is
 * walked in its enclosing cube's order, missing cells skipped). perm[i] is
 * the raster token index placed at position i. Requires 1 <= ndim <= 4,
 * every grid[a] >= 1, prefix >= 0, n = prefix + prod(grid) <= 2^31 - 1 and
 * ndim * bits(max grid) <= 63; else PISA_ERR_SHAPE (PISA_ERR_NULL for a NULL
 * pointer). The caller owns perm.
 */
pisa_status_t pisa_z_order(const int64_t *grid, int32_t ndim, int64_t prefix, int32_t *perm,
                           int64_t n);

/*
 * pisa_reorder_gather: out[b,h,i,:] = x[b, perm[i], h, :]: tokens gathered
 * into the order perm while [B,T,H,D] becomes [B,H,T,D] (shape.seq_len = T,
 * shape.heads = H, shape.head_dim = D, shape.dtype the element type; the
 * other fields are checked as for the operator). perm: int32 [T] (device),
 * normally a permutation of [0, T); a position whose perm entry is outside
 * [0, T) receives zeros. x and out are device buffers that must not overlap.
 *
 * pisa_reorder_scatter: the inverse, y[b, perm[i], h, :] = o[b,h,i,:]
 * ([B,H,T,D] back to raster-order [B,T,H,D]); positions whose perm entry is
 * outside [0, T) are not written. With a permutation, scatter(gather(x)) = x
 * bit for bit.
 */
pisa_status_t pisa_reorder_gather(const pisa_shape_t *shape, const int32_t *perm, const void *x,
                                  void *out, void *stream);
pisa_status_t pisa_reorder_scatter(const pisa_shape_t *shape, const int32_t *perm, const void *o,
                                   void *y, void *stream);

/*
 * Backward of pisa_attn_fwd ("Piecewise-Taylor-Attention" README: the
 * trainable regime, gradients through both the exact and the approximate
 * branch with the block selection detached; PISA §3.2 Eqs. 3-5 and §3.3
 * Eqs. 9-10 for the function being differentiated).
 *
 * pisa_attn_bwd writes dq, dk, dv = the gradients of L = sum dout . o with
 * respect to q, k and v, where o is pisa_attn_fwd's output for the same
 * shape, params, q, k, v, stats, idx and wgate. idx and the gate (which pairs
 * of wgate hold 0) are constants of the differentiation; every statistic the
 * forward derives from q, k, v (block means, V-hat, H, and for second order
 * the pooled q^2 and the key variance inside w_ij) is differentiated through.
 * Arguments:
 *   q, k, v, o, dout  [B,H,T,D] in the shape's dtype (o as the forward wrote
 *                     it: it enters only through delta_t = dout_t . o_t);
 *   stats             as pisa_block_stats wrote them for q, k, v; reads kbar,
 *                     vsum, hsum (and q2bar, ksig2 if second_order);
 *   idx, wgate        as passed to pisa_attn_fwd;
 *   row_stats         NULL, or the row_stats pisa_attn_fwd wrote with this o:
 *                     bf16 inputs then take each row's lse and c from it
 *                     instead of re-scoring the row's exact and virtual
 *                     pairs (fp32 inputs recompute them either way);
 *   dq, dk, dv        [B,H,T,D] outputs in the shape's dtype; they must not
 *                     alias each other, the inputs, row_stats or the workspace;
 *   workspace         caller-owned device memory of at least
 *                     pisa_attn_bwd_workspace_bytes(shape) bytes (per-row
 *                     statistics, the selection bitmask, per-block partial
 *                     gradients, dH); contents on entry are ignored and on
 *                     return unspecified.
 * params->phase_mask must be 0 (PISA_ERR_UNSUPPORTED otherwise). fp32 inputs:
 * fp32 arithmetic. bf16 inputs: every product on bf16 matrix cores with fp32
 * accumulation; the intermediate weights (P, dS and the virtual tokens'
 * A, dlam) and the fp32 statistics (kbar, V-hat, H) enter as bf16 hi + lo
 * pairs (about 16 significant bits). Each gradient is rounded once to the
 * output dtype. Deterministic: no floating-point atomics.
 */
size_t pisa_attn_bwd_workspace_bytes(const pisa_shape_t *shape);
pisa_status_t pisa_attn_bwd(const pisa_shape_t *shape, const pisa_params_t *params,
                            const void *q, const void *k, const void *v, const void *o,
                            const void *dout, const pisa_stats_t *stats, const int32_t *idx,
                            const float *wgate, const float *row_stats, void *dq, void *dk,
                            void *dv, void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PISA_H_ */
