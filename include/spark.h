/*
 * spark.h -- C ABI of libspark, a gfx950 (MI355X) implementation of one
 * Spark-Attn block-sparse attention layer: Spark-Reblock, block top-k,
 * Spark-Reweight summaries and the fused exact + compressed attention.
 *
 * The operations follow the pages of the "Spark-H3: Adaptive Block Sparse
 * Attention for MiniMax-H3" blog (zechengtang.github.io/Spark-H3), cited
 * below as [blog] with the section name, plus the comfy.icu Spark-H3 package
 * README ([readme], "Spark-Attn" section) and the comfyui-wiki.com Spark-H3
 * news item ([news], "What Spark-Attn changes").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor argument is a DEVICE pointer into memory the caller owns
 *    (allocated e.g. by PyTorch).  The library never allocates, frees or
 *    synchronises; scratch memory comes only through (ws, ws_bytes), sized
 *    with spark_workspace_bytes().  Pointers must be 16-byte aligned.
 *  - Calls are asynchronous and ordered on `stream` (a hipStream_t; NULL is
 *    the null stream).  The library keeps no state between calls.
 *  - Results are deterministic: every reduction runs in a fixed order, so
 *    the same inputs give bit-identical outputs on every call, whatever
 *    the workspace held before; a head's outputs do not depend on how many
 *    heads the call holds.
 *  - Return value: SPARK_OK (0) or a negative spark_status.  All argument
 *    checks run before anything is enqueued, so a failed call enqueues
 *    nothing.  A failed launch returns SPARK_E_HIP.  spark_last_error()
 *    gives a message for the calling thread's last failure.  No C++
 *    exception crosses this ABI.
 *  - Shapes: H >= 1 heads, N >= 1 tokens, head dim d in {64, 128}, block
 *    size 1 <= block <= 128 (N need not be a multiple of block: the last
 *    block holds r = N - (n_b - 1) * block tokens).  n_b = ceil(N / block),
 *    Np = n_b * block.  dtype is SPARK_F32 or SPARK_BF16 for q, k, v and
 *    everything derived from them in that dtype; moments, means, summaries,
 *    scores and biases are always fp32.
 *  - Layouts (row-major, contiguous):
 *      q, k, v, out      [H, N, d]          dtype
 *      perm_q, perm_k    [H, N]             int32, perm[p] = original token id
 *      q_p, k_p          [H, Np, d]         dtype, rows >= N written as 0
 *      v_pt              [H, n_b, d, block] dtype, block-transposed gathered V:
 *                        v_pt[h][B][c][j] = v[h][perm_k[h][B*block + j]][c],
 *                        0 where B*block + j >= N
 *      qbar, kbar        [H, n_b, d]        fp32 block means over real rows
 *      anchor            [H, d]             fp32
 *      scores            [H, n_b, n_b]      fp32
 *      idx               [H, n_b, topk]     int32, ascending per row
 *      ksum, vsum        [H, n_b, d]        fp32
 *      bias              [H, n_b]           fp32
 *      M, W              [count, d, d]      fp32
 */
#ifndef SPARK_H
#define SPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* spark_stream_t; /* == hipStream_t */

typedef enum spark_status {
  SPARK_OK = 0,
  SPARK_E_ARG = -1,         /* null / misaligned pointer, bad count or flag  */
  SPARK_E_SHAPE = -2,       /* H, N, block, topk out of range                */
  SPARK_E_DTYPE = -3,       /* dtype not SPARK_F32 / SPARK_BF16              */
  SPARK_E_UNSUPPORTED = -4, /* d not in {64, 128}                            */
  SPARK_E_WORKSPACE = -5,   /* ws too small or null                          */
  SPARK_E_HIP = -6          /* a HIP launch failed                           */
} spark_status;

typedef enum spark_dtype { SPARK_F32 = 0, SPARK_BF16 = 1 } spark_dtype;

/* flags: token layout (how blocks are formed) */
#define SPARK_LAYOUT_REBLOCK 0x0u   /* Spark-Reblock partition ([blog] 01 / Method: Spark-Reblock) */
#define SPARK_LAYOUT_IDENTITY 0x1u  /* consecutive tokens: the fixed-partition BSA baseline          */
#define SPARK_LAYOUT_GIVEN 0x2u     /* perm_q / perm_k are inputs                                   */
#define SPARK_LAYOUT_Q_REUSE_K 0x3u /* the key partition also groups the queries ([news] Workflows) */
#define SPARK_LAYOUT_MASK 0x3u
/* flags: compressed-branch estimator */
#define SPARK_SUMMARY_REWEIGHT 0x0u /* Spark-Reweight ([blog] 02 / Method: Spark-Reweight)          */
#define SPARK_SUMMARY_MEAN 0x4u     /* uniform block means, no bias (BSA / Sol-Attn estimator)      */
/* flags: context/sink tokens ([blog] 01 / Method: Spark-Reblock: context/sink
 * tokens stay exact and lie outside the video-block Top-K budget).  Tokens
 * [n_anchor, N) of every head are context tokens, [0, n_anchor) video tokens:
 *   - only the video tokens are partitioned, pooled, scored, routed and
 *     summarised: n_b = ceil(n_anchor / block) video blocks, and topk,
 *     qbar, kbar, idx, ksum, vsum, bias all count video blocks;
 *   - the n_c = ceil((N - n_anchor) / block) context blocks follow the video
 *     blocks in q_p, k_p and v_pt (context tokens in original order), so
 *     those hold n_t = n_b + n_c blocks: q_p, k_p [H, n_t * block, d],
 *     v_pt [H, n_t, d, block];
 *   - perm_q / perm_k keep the context tokens in place (perm[p] = p for
 *     p >= n_anchor); the moments still use all N tokens;
 *   - every video query attends exactly to all context keys besides its
 *     selected blocks; a context query's row is exact dense attention over
 *     all N keys.
 * Honoured by spark_reblock, spark_select, spark_summarize, spark_attn,
 * spark_layer and spark_workspace_bytes; the stage entry points and
 * spark_diagnostics reject it (SPARK_E_UNSUPPORTED).  With n_anchor = N it
 * changes nothing. */
#define SPARK_CONTEXT_EXACT 0x8u
/* flags: fp8 attention logits ([blog] 03 / Evaluation: Benchmark Results, the
 * DiT's FP8 runs; the pages give no further detail).  Every attention logit
 * q . k is computed from OCP E4M3 operands: each query row, each key block
 * (block rows) and each group of `block` consecutive summary keys is scaled
 * by the smallest power of two s with max |x| <= 448 s and rounded to the
 * nearest E4M3 value (ties to even); the logit is s_q s_k (q8 . k8).  P and
 * V keep the bf16 path.  Supported for bf16, d = 128, block = 128 (the
 * spark_attn / spark_layer kernels); SPARK_E_UNSUPPORTED otherwise, and
 * from spark_diagnostics. */
#define SPARK_EXACT_FP8 0x10u
/* flags: schedule choice for the bf16, d = 128, block = 128 attention of
 * spark_attn, spark_attn_noalloc and spark_layer (other entry points ignore
 * it).  By default, where the layer has no context tokens and the tiles fit
 * in LDS, one workgroup runs two adjacent query blocks and loads the key
 * blocks both selected once for both; this flag keeps one query block per
 * workgroup.  Both compute the same quantity; the outputs differ only in
 * fp32 rounding order (the tiles are visited in another order). */
#define SPARK_ATTN_ONE_BLOCK 0x20u

typedef struct spark_args {
  int32_t H;        /* heads                                                  */
  int32_t N;        /* tokens per head                                        */
  int32_t d;        /* head dim, 64 or 128                                    */
  int32_t block;    /* tokens per block, 1..128                               */
  int32_t dtype;    /* spark_dtype of q, k, v                                 */
  int32_t n_anchor; /* the anchor averages query rows [0, n_anchor); 1..N     */
  uint32_t flags;   /* SPARK_LAYOUT_* | SPARK_SUMMARY_* | SPARK_CONTEXT_EXACT |
                       SPARK_EXACT_FP8 | SPARK_ATTN_ONE_BLOCK */
  int32_t reserved; /* must be 0                                              */
} spark_args;

typedef enum spark_op {
  SPARK_OP_REBLOCK = 0,
  SPARK_OP_SELECT = 1,
  SPARK_OP_SUMMARIZE = 2,
  SPARK_OP_ATTN = 3,
  SPARK_OP_SPLIT = 4,   /* spark_split on 2*H trees of N tokens */
  SPARK_OP_LAYER = 5
} spark_op;

/* ---- utilities --------------------------------------------------------- */

/* Library version, major * 10000 + minor * 100 + patch. */
int spark_version(void);

/* Human-readable name of a status code (static string). */
const char* spark_status_string(int status);

/* Message of the calling thread's last failed call ("" if none). */
const char* spark_last_error(void);

/* ceil(N / block), or a negative status for bad arguments. */
int spark_block_count(int32_t N, int32_t block);

/* Exact-branch budget for a density ratio: the Top-K of [blog] 01 / Method:
 * Spark-Reblock covers "the top 10% of video key-value blocks"; read as the
 * smallest block count covering the ratio, min(n_blocks, max(1,
 * ceil(ratio * n_blocks - 1e-9))).  Negative status for n_blocks < 1 or a
 * non-finite ratio. */
int spark_topk_from_ratio(double ratio, int32_t n_blocks);

/* Bytes of workspace `op` needs for these arguments (topk is used by
 * SPARK_OP_ATTN and SPARK_OP_LAYER only).  0 if none; (size_t)-1 for
 * invalid arguments. */
size_t spark_workspace_bytes(const spark_args* args, int op, int32_t topk);

/* ---- the four steps of the layer ---------------------------------------- */

/* Spark-Reblock ([blog] 01 / Method: Spark-Reblock, the d_Q equation and the
 * hierarchical partitioner) followed by the permutation gather and block
 * pooling.  Per head:
 *   M_K = E[k k^T], M_Q = E[q q^T] over all N tokens (uncentred);
 *   queries are whitened by M_K^{1/2}, keys by M_Q^{1/2}, and normalised,
 *   so that x^_i . x^_j = 1 - d_Q(i, j);
 *   each side is split level by level (two-pole capacity bisection: pole A
 *   farthest from the group centroid, pole B farthest from A, score
 *   s = x^.x^_A - x^.x^_B, the left child takes the ceil(blocks/2)*block
 *   largest scores, ties to the lower token id) until every leaf is one
 *   block; leaves in depth-first left-first order, ids ascending inside a
 *   leaf, a short remainder block last;
 *   q_p, k_p, v_pt are the gathered tokens, qbar / kbar the block means;
 *   anchor = mean of query rows [0, n_anchor) in original order (the
 *   representative query of [blog] 02 / Method: Spark-Reweight, one per head
 *   as in [news]).
 * flags & SPARK_LAYOUT_MASK: REBLOCK computes perm_q/perm_k (outputs);
 * Q_REUSE_K splits the keys only (whitened by M_Q^{1/2} as above; the
 * reblock_layout=q_reuse_k setting of the [news] page's Workflows section)
 * and writes that permutation to both perm_k and perm_q; IDENTITY writes
 * perm = 0..N-1; GIVEN reads perm_q/perm_k (inputs, each a permutation of
 * 0..N-1 per head; not checked; with SPARK_CONTEXT_EXACT only entries
 * [0, n_anchor) are read, each a permutation of 0..n_anchor-1).
 * q_p and anchor may be NULL (not written).  ws: spark_workspace_bytes(args,
 * SPARK_OP_REBLOCK, 0) bytes (0 for IDENTITY and GIVEN). */
int spark_reblock(const spark_args* args, const void* q, const void* k, const void* v,
                  int32_t* perm_q, int32_t* perm_k, void* q_p, void* k_p, void* v_pt,
                  float* qbar, float* kbar, float* anchor, void* ws, size_t ws_bytes,
                  spark_stream_t stream);

/* Block scoring and fixed Top-K routing ([blog] Discussion: blocks are scored
 * from block-level means; Top-K budget per query block):
 *   S[h][A][B] = qbar[h][A] . kbar[h][B] / sqrt(d),
 *   idx[h][A] = the topk blocks B with the largest S (ties: lower B; NaN
 *   ranks below -inf), stored in ascending B order.
 * If scores_in is non-NULL the scores are read from it instead (qbar, kbar
 * may then be NULL).  scores_out (nullable) receives the scores used.
 * 1 <= topk <= n_b. */
int spark_select(const spark_args* args, const float* qbar, const float* kbar,
                 const float* scores_in, int32_t topk, int32_t* idx, float* scores_out,
                 spark_stream_t stream);

/* Compressed-branch summaries of every key block B ([blog] 02 / Method:
 * Spark-Reweight; [readme] Spark-Attn: different weights per token of a tail
 * block).  REWEIGHT: t_j = anchor . k_j / sqrt(d) for j in B,
 *   w = softmax_B(t), ksum_B = sum w_j k_j, vsum_B = sum w_j v_j,
 *   bias_B = log sum_j exp(t_j) - log n_B - anchor . ksum_B / sqrt(d),
 * so exp(anchor . ksum_B / sqrt(d) + bias_B) is the block's mean exponential.
 * MEAN (flags & SPARK_SUMMARY_MEAN): uniform means, bias 0; anchor unused
 * (may be NULL). */
int spark_summarize(const spark_args* args, const void* k_p, const void* v_pt,
                    const float* anchor, float* ksum, float* vsum, float* bias,
                    spark_stream_t stream);

/* Fused two-branch attention ([blog] 01 / Method: Spark-Reblock, BSA(Q_A)
 * equations: one row-wise softmax over the selected blocks' exact keys and,
 * for every other block B, its summary repeated n_B times), i.e. for query
 * row i of block A
 *   o_i = (sum_{B in S_A, j in B} e^{q_i.k_j/sqrt d} v_j
 *          + sum_{B not in S_A} n_B e^{q_i.ksum_B/sqrt d + bias_B} vsum_B)
 *         / (the same sums without the values),
 * computed with an online softmax, then scattered: out[h][perm_q[h][p]] =
 * o_p.  If perm_q is NULL the output stays in permuted order and `out` is
 * [H, Np, d] (padding rows written as 0; Np = n_t * block with
 * SPARK_CONTEXT_EXACT).  idx rows must be strictly
 * ascending block ids in [0, n_b) (not checked on the device).
 * ws: spark_workspace_bytes(args, SPARK_OP_ATTN, topk) bytes. */
int spark_attn(const spark_args* args, const void* q_p, const void* k_p, const void* v_pt,
               const int32_t* idx, int32_t topk, const float* ksum, const float* vsum,
               const float* bias, const int32_t* perm_q, void* out, void* ws, size_t ws_bytes,
               spark_stream_t stream);

/* spark_attn without a workspace argument, for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, results (bit for bit) and
 * errors as spark_attn; its scratch is a file-scope device array of
 * spark_attn_noalloc_scratch_bytes() bytes (64 MiB) that each GPU the
 * library runs on holds until the process ends.  Arguments whose
 * spark_workspace_bytes(args, SPARK_OP_ATTN, topk) exceeds that size are
 * rejected with SPARK_E_WORKSPACE before anything is enqueued (the 768p
 * layer needs about 42 MB; E4M3 logits at that size do not fit).  The first
 * call made with a device current looks up that device's copy of the array;
 * no call allocates or frees memory.  All calls on one GPU share its array:
 * calls that overlap on one GPU (other streams, other host threads) race on
 * it and must be serialised by the caller. */
int spark_attn_noalloc(const spark_args* args, const void* q_p, const void* k_p, const void* v_pt,
                       const int32_t* idx, int32_t topk, const float* ksum, const float* vsum,
                       const float* bias, const int32_t* perm_q, void* out, spark_stream_t stream);

/* Bytes of the scratch array spark_attn_noalloc works in (per GPU). */
size_t spark_attn_noalloc_scratch_bytes(void);

/* The whole layer: spark_reblock -> spark_select -> spark_summarize ->
 * spark_attn, with every intermediate in ws
 * (spark_workspace_bytes(args, SPARK_OP_LAYER, topk) bytes). */
int spark_layer(const spark_args* args, const void* q, const void* k, const void* v,
                int32_t topk, void* out, void* ws, size_t ws_bytes, spark_stream_t stream);

/* ---- the stages of spark_reblock, exposed for composition and testing ---- */

/* Second moments M_Q[h] = (1/N) sum_i q_i q_i^T and M_K[h] likewise for k
 * ([blog] 01 / Method: Spark-Reblock, the M_K = E[k k^T] of the d_Q
 * equation).  anchor (nullable) as in spark_reblock.  ws:
 * spark_workspace_bytes(args, SPARK_OP_REBLOCK, 0) is enough. */
int spark_moments(const spark_args* args, const void* q, const void* k, float* MQ, float* MK,
                  float* anchor, void* ws, size_t ws_bytes, spark_stream_t stream);

/* Symmetric PSD square roots W[i] = M[i]^{1/2} of `count` d x d matrices
 * ([blog] 01 / Method: Spark-Reblock, M_K^{1/2}).  Coupled Newton-Schulz in
 * fp32 after scaling by the Frobenius norm (the input is symmetrised first);
 * an all-zero M gives W = 0, a non-finite M gives NaN.  ws, ws_bytes:
 * unused (the iteration runs in on-chip memory); may be NULL and 0. */
int spark_msqrt(int32_t count, int32_t d, const float* M, float* W, void* ws, size_t ws_bytes,
                spark_stream_t stream);

/* Whitening: xhat[t][i] = W[t] x[t][i] / ||W[t] x[t][i]|| (0 if the norm is
 * 0), for `count` matrices of N rows (x, xhat [count, N, d] in dtype, W
 * [count, d, d] fp32).  Uses args->N, d, dtype. */
int spark_whiten(const spark_args* args, int32_t count, const void* x, const float* W,
                 void* xhat, spark_stream_t stream);

/* The hierarchical partitioner alone on `count` trees of given vectors xhat
 * [count, N, d] (dtype), taken as they are (not normalised), writing perm
 * [count, N].  Uses args->N, d, block, dtype.  Arithmetic is fp32 with
 * deterministic reduction order, so integer-valued inputs whose sums stay
 * below 2^24 give exactly the result of the rule in exact arithmetic.
 * ws: spark_workspace_bytes(args with H = ceil(count / 2), SPARK_OP_SPLIT, 0). */
int spark_split(const spark_args* args, int32_t count, const void* xhat, int32_t* perm,
                void* ws, size_t ws_bytes, spark_stream_t stream);

/* Permutation gather and block pooling of one side ([blog] 01 / Method:
 * Spark-Reblock, token IDs track membership through the tree): for every
 * head, x_p (nullable) = x[perm] padded to Np rows, x_pt (nullable) the
 * block-transposed layout of v_pt, xbar (nullable) the fp32 block means over
 * real rows. */
int spark_gather(const spark_args* args, const void* x, const int32_t* perm, void* x_p,
                 void* x_pt, float* xbar, spark_stream_t stream);

/* E4M3 quantisation as SPARK_EXACT_FP8 applies it: `rows` rows of d values
 * (x: SPARK_BF16 or SPARK_F32 per dtype, d in {64, 128}) in consecutive
 * groups of `group` rows (the last may be short); group g is scaled by the
 * smallest power of two s_g with max |x| <= 448 s_g (s_g = 1 for an all-zero
 * group) and x / s_g is rounded to the nearest OCP E4M3 value, ties to even.
 * Writes x8 [rows, d] bytes (4-byte aligned) and scales [ceil(rows / group)]
 * fp32 (the s_g).  Device pointers, enqueued on the stream. */
int spark_quant_e4m3(int32_t rows, int32_t d, int32_t group, int32_t dtype, const void* x,
                     uint8_t* x8, float* scales, spark_stream_t stream);

/* ---- test hooks: the splitter's selection rules on caller values -------- */

/* One capacity partition, as every split of spark_reblock performs it
 * ([blog] 01 / Method: Spark-Reblock, the partitioner paragraph: each group
 * is split by the distance while the child capacities are enforced; the
 * two-pole rule and its tie rules are this library's reading).  For each of
 * `count` rows of n positions (s: fp32 scores, ids_in: int32 token ids, both
 * [count, n]; within a row the ids must be ascending, as in every group of
 * the splitter, since ties are ranked by position): the left child is the
 * c_L = ceil(ceil(n / block) / 2) * block positions first in (s descending,
 * id ascending) order, where -0 equals +0 and NaN ranks after every number;
 * ids_out [count, n] receives the left child's ids, then the right child's,
 * each in input order.  Runs the kernels the splitter's top level uses for a
 * group of that many blocks.  ws: spark_debug_partition_ws_bytes(count, n,
 * block) bytes (SPARK_E_WORKSPACE if smaller).  Device pointers, 16-byte
 * aligned; enqueued on the stream. */
size_t spark_debug_partition_ws_bytes(int32_t count, int32_t n, int32_t block);
int spark_debug_partition_level(int32_t count, int32_t n, int32_t block, const float* s,
                                const int32_t* ids_in, int32_t* ids_out, void* ws, size_t ws_bytes,
                                spark_stream_t stream);

/* The pole choice of every split (same passage and reading as above: pole A
 * is the member farthest from the group centroid, pole B the member
 * farthest from A, both an argmin of a dot product): for each of `count`
 * rows of n fp32 values vals [count, n] with int32 ids [count, n] (ids >= 0),
 * out[row] = the id of the minimum value, where -0 equals +0, NaN ranks
 * after every number and equal values go to the lower id; the same 64-bit
 * (value key, id) ordering and wave reduction as the splitter's argmin
 * passes.  Device pointers, 16-byte aligned; enqueued on the stream. */
int spark_debug_argmin(int32_t count, int32_t n, const float* vals, const int32_t* ids, int32_t* out,
                       spark_stream_t stream);

/* ---- measurement helper (not part of the layer) -------------------------- */

/* Enqueues one launch of a register-only bf16 matrix-core loop
 * (v_mfma_f32_32x32x16_bf16, four independent accumulator chains per wave,
 * `workgroups` workgroups of 4 waves, `iters` iterations) and returns the
 * floating-point operations it performs, so that the caller's event timing
 * of the launch gives the sustained bf16 MFMA rate of the part (the roofline
 * peak the attention kernel is compared against).  sink: device buffer of
 * workgroups * 256 floats that is never written in practice.  Returns -1 on
 * bad arguments or a failed launch (spark_last_error() says why). */
double spark_mfma_peak_probe(int32_t workgroups, int32_t iters, float* sink, spark_stream_t stream);

/* ---- routing diagnostics (outside the layer; dense cost) ---------------- */

/* Per query row p of the permuted order (q_p, k_p as written by
 * spark_reblock; idx, ksum, bias as for spark_attn):
 *   recall[h][p]  = dense softmax mass of row p on the exact keys of its
 *                   query block's selected blocks (the attention-mass recall
 *                   compared between reblocked and fixed blocks in [blog]
 *                   01 / Method: Spark-Reblock);
 *   logmass[h][p] = | log sum over unselected blocks' keys of e^{q.k/sqrt d}
 *                   - log sum over unselected blocks of
 *                     n_B e^{q.ksum_B/sqrt d + bias_B} |
 *                   (the log-mass error of [blog] 02 / Method: Spark-Reweight;
 *                   0 when every block is selected).
 * recall, logmass: [H, N] fp32, either may be NULL (not both).  Reads every
 * key for every query: O(H N^2 d) work, fp32 accumulation. */
int spark_diagnostics(const spark_args* args, const void* q_p, const void* k_p, const int32_t* idx,
                      int32_t topk, const float* ksum, const float* bias, float* recall,
                      float* logmass, spark_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARK_H */
