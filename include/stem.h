/*
 * stem.h - C ABI of the Stem block-sparse causal prefill path on MI355X.
 *
 * The method ("Stem: Rethinking Causal Information Flow in Sparse Attention",
 * arXiv 2603.06274) replaces the prefill attention of one layer: queries,
 * keys and values of a prompt go in, the attention output comes out
 * (gist.science/es "Resumen tecnico" section 1; gist.science/fr "Resume
 * technique" section 1).  Its implementation runs in three stages
 * (gist.science/es "Implementacion", gist.science/nl "Implementatie",
 * gist.science/fr section 2.C):
 *   1. downsample Q, K and the V magnitude to block level   -> stem_pool
 *   2. fix a budget per query block (Token Position-Decay)  -> stem_plan
 *   3. keep the top blocks of the Output-Aware Metric and    -> stem_score,
 *      run exact softmax attention over them only               stem_select,
 *                                                               stem_sparse_attn
 *
 * Conventions shared by every call:
 *   - Tensors are dense, contiguous and token-major ("THD"): Q is
 *     [T, Hq, d], K and V are [T, Hkv, d]; query head h reads KV head
 *     h / (Hq / Hkv).  A packed batch of sequences is described by
 *     cu_seqlens (sequence s owns tokens [cu_seqlens[s], cu_seqlens[s+1])).
 *   - Block j of sequence s covers its tokens [j*B, min((j+1)*B, len_s));
 *     a sequence has ceil(len_s / B) blocks and the last one may be
 *     partial.  Blocks are numbered globally in sequence order
 *     ("global block"); block numbers stored in selection lists are local
 *     to their sequence.
 *   - Ownership: the caller allocates and frees every buffer.  The library
 *     never allocates, frees or synchronises and keeps no global state.
 *   - Device calls are asynchronous on the given stream (a hipStream_t
 *     passed as void*; NULL is the default stream).  All host-side checks
 *     happen before any launch: on a negative return nothing was launched
 *     and no output was written.  A launch failure returns STEM_EHIP; a
 *     fault inside a kernel surfaces at the caller's next synchronisation.
 *   - Pointer alignment: Q, K, V, O and the pooled buffers must be 16-byte
 *     aligned; all other device buffers 4-byte aligned.
 *   - No C++ exception crosses this interface.
 */
#ifndef STEM_H
#define STEM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  STEM_OK = 0,
  STEM_EINVAL = -1,        /* a null pointer, a bad size or inconsistent arguments */
  STEM_EUNSUPPORTED = -2,  /* valid but not implemented (head_dim, block, dtype, size limits) */
  STEM_EHIP = -3,          /* the HIP runtime reported an error at launch */
  STEM_ESPACE = -4         /* the caller's host buffer for the plan is too small */
} stem_status;

typedef enum { STEM_F32 = 0, STEM_BF16 = 1 } stem_dtype;

/* Shape of the position-dependent budget (see stem_params). */
typedef enum {
  STEM_BUDGET_EXP = 0,              /* exponential decay (rho0, tau)                   */
  STEM_BUDGET_LINEAR = 1,           /* linear k_start -> mu * k_start, k_start in blocks */
  STEM_BUDGET_LINEAR_FRACTION = 2   /* the same ramp, k_start a fraction of the causal
                                       blocks of each query block                      */
} stem_budget_mode;

/* Which block metric stem_score writes (see stem_score). */
typedef enum {
  STEM_METRIC_OUTPUT_AWARE = 0,  /* softmax_j(s_ij) * w_j                      */
  STEM_METRIC_ADDITIVE = 1,      /* s_ij + beta * max(0, log(w_j^2))            */
  STEM_METRIC_ROUTING = 2        /* softmax_j(s_ij): attention score alone      */
} stem_metric_mode;

/* How the block V magnitude is pooled (the method's metric needs one value
 * per key block).  MEAN: mean over the block's tokens of ||v_t||_2.
 * MAX: the maximum of ||v_t||_2 over the block's tokens. */
typedef enum { STEM_VNORM_MEAN = 0, STEM_VNORM_MAX = 1 } stem_vnorm_mode;

/* Shape of one prefill layer. */
typedef struct stem_problem {
  int32_t num_seqs;             /* >= 1 */
  const int32_t *cu_seqlens;    /* host array [num_seqs + 1]; cu[0] = 0, non-decreasing */
  int32_t num_q_heads;          /* Hq >= 1 */
  int32_t num_kv_heads;         /* Hkv >= 1, divides Hq */
  int32_t head_dim;             /* d: 64 or 128 */
  int32_t block;                /* B: 64 or 128 */
  int32_t dtype;                /* stem_dtype of Q, K and V */
} stem_problem;

/* Token Position-Decay budget (gist.science/es 2.A, gist.science/fr 2.A: a
 * high budget for early query positions decaying to a lower one later).
 * For local query block i of a sequence with nb blocks, k_dyn(i) is
 *   STEM_BUDGET_EXP (decay shape of the shd-paper.top method detail):
 *     max(k_min, ceil(rho0 * exp(-i / tau) * (i + 1)))
 *   STEM_BUDGET_LINEAR (the gist.science pages' linear interpolation from
 *   k_start to k_end = mu * k_start over the sequence's query blocks):
 *     max(k_min, ceil(k_start * (1 - f) + mu * k_start * f)), f = i / (nb - 1)
 *   STEM_BUDGET_LINEAR_FRACTION (the same ramp read as a share of the causal
 *   blocks: row i keeps that fraction of its i + 1 key blocks):
 *     max(k_min, ceil((k_start * (1 - f) + mu * k_start * f) * (i + 1)))
 * evaluated in fp64 (f = 0 when nb = 1), and the kept count is
 *   k_i = i + 1                                if i < sink_blocks
 *       = min(i + 1, sink_blocks + 1 + k_dyn(i)) otherwise
 * so the first sink_blocks blocks (initial tokens are the anchors every
 * later token aggregates, gist.science/es section 1) and the diagonal block
 * are always kept and k_dyn further blocks are chosen by the metric.
 * rho0 = 0 (or mu = 1) gives a uniform budget. */
typedef struct stem_params {
  int32_t sink_blocks;          /* S >= 0 */
  int32_t k_min;                /* >= 0 */
  double rho0;                  /* >= 0, finite (EXP) */
  double tau;                   /* > 0, in blocks (EXP) */
  int32_t budget_mode;          /* stem_budget_mode */
  int32_t metric_mode;          /* stem_metric_mode */
  double k_start;               /* LINEAR: >= 0, finite, in blocks;
                                   LINEAR_FRACTION: in [0, 1], a fraction */
  double mu;                    /* in [0, 1] (LINEAR, LINEAR_FRACTION) */
  double beta;                  /* >= 0, finite (ADDITIVE metric) */
} stem_params;

/* Sizes and offsets computed by stem_plan.  The caller passes it back,
 * unchanged, to every device call together with the uploaded plan blob. */
typedef struct stem_plan_info {
  int32_t magic;                    /* STEM_PLAN_MAGIC */
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim, block, dtype;
  int32_t sink_blocks;
  int32_t kmax;                     /* max_i k_i: third extent of idx */
  int32_t max_seq_blocks;           /* max_s ceil(len_s / B) */
  int32_t metric_mode;              /* stem_metric_mode */
  int32_t reserved;
  double beta;                      /* ADDITIVE metric weight */
  int64_t total_tokens;             /* T */
  int64_t total_blocks;             /* nbT = sum_s ceil(len_s / B) */
  int64_t score_elems_per_head;     /* sum_s nb_s (nb_s + 1) / 2 */
  int64_t executed_blocks_per_head; /* sum over query blocks of k_i */
  int64_t plan_bytes;               /* size of the plan blob */
  /* byte offsets of the arrays inside the plan blob */
  int64_t off_cu_seqlens;  /* int32 [num_seqs + 1] */
  int64_t off_cu_blocks;   /* int32 [num_seqs + 1] first global block of each sequence */
  int64_t off_tri;         /* int64 [num_seqs + 1] start of each sequence's score triangle in a head */
  int64_t off_blk_seq;     /* int32 [nbT] sequence of each global block */
  int64_t off_budget;      /* int32 [nbT] k_i of each global query block */
  int64_t off_order;       /* int32 [nbT] global query blocks, most work first */
} stem_plan_info;

#define STEM_PLAN_MAGIC 0x5354454d

/* stem_plan - host only, touches no HIP API.
 * Validates the problem and parameters, fills *info and, when plan_host is
 * not NULL, writes the plan blob (info->plan_bytes bytes) there.  The
 * caller copies the blob to device memory (16-byte aligned) and passes that
 * copy as plan_dev to the device calls.  Call with plan_host = NULL first to
 * learn plan_bytes.  Returns STEM_ESPACE if capacity < plan_bytes.
 * Size limits (STEM_EUNSUPPORTED beyond them): at most 4096 blocks in one
 * sequence (the selection keeps a row's candidates in one wavefront's
 * registers), T < 2^31 tokens, nbT < 2^30 blocks and Hq * nbT < 2^31. */
int stem_plan(const stem_problem *problem, const stem_params *params,
              stem_plan_info *info, void *plan_host, int64_t capacity);

/* stem_pool - block downsampling (stage 1).
 *   qbar [Hq, nbT, d]  f32: mean of Q over each block's tokens
 *   kbar [Hkv, nbT, d] f32: mean of K over each block's tokens
 *   vnorm [Hkv, nbT]   f32: block V magnitude (mode, see stem_vnorm_mode)
 * q, k, v have the plan's dtype. */
int stem_pool(const stem_plan_info *info, const void *plan_dev,
              const void *q, const void *k, const void *v,
              float *qbar, float *kbar, float *vnorm, int32_t vnorm_mode,
              void *stream);

/* stem_score - Output-Aware Metric per (query block, causal key block)
 * (gist.science/es 2.B; gist.science/fr 2.B: routing relevance combined
 * with the magnitude of the values).  For query head h, sequence s, local
 * query block i and local key block j <= i, with s_ij = qbar_i . kbar_j / sqrt(d):
 *   OUTPUT_AWARE  m_ij = softmax over j in [0, i] of s_ij, times vnorm_j
 *   ADDITIVE      m_ij = s_ij + beta * max(0, log(vnorm_j^2))  (the pages'
 *                 displayed formula, gist.science/es 2.B equation)
 *   ROUTING       m_ij = softmax over j in [0, i] of s_ij (routing alone,
 *                 the criterion the pages argue against, es section 1)
 * (mode and beta from the plan)
 * scores is f32 [Hq, score_elems_per_head]: for each head the sequences'
 * lower triangles one after another (plan off_tri), row i of a sequence
 * starting i (i + 1) / 2 elements into its triangle. */
int stem_score(const stem_plan_info *info, const void *plan_dev,
               const float *qbar, const float *kbar, const float *vnorm,
               float *scores, void *stream);

/* stem_score_antidiag - the metric of stem_score with block logits taken from
 * anti-diagonal samples of the token logits instead of the pooled blocks
 * (gist.science/fr, "Resume technique" 2.C step 1: block metrics computed
 * with anti-diagonal sampling).  For stride S (a power of two, 1 <= S <= B),
 * each sequence's tokens form groups of S positions; the sample of query
 * group r and key group c is the mean of q.k / sqrt(d) over the pairs
 * (query rS + S-1-u, key cS + u), u = 0..S-1, whose tokens exist and whose
 * key is not after the query; the block logit t_ij is the log of the mean of
 * exp(sample) over the samples of query block i and key block j (-inf if
 * there are none) and takes the place of s_ij in the metric mode of the plan.
 * A row whose logits are all -inf gets 0 in the softmax forms.  S = 1 gives
 * the exact log-mean-exp of each block pair's causal token logits.
 *   q [T, Hq, d], k [T, Hkv, d]: the plan's dtype, 16-byte aligned; vnorm
 *   [Hkv, nbT] f32 from stem_pool; scores as for stem_score (fully
 *   overwritten).  STEM_EINVAL for a bad stride; for bf16 plans
 *   STEM_EUNSUPPORTED when the work bound Hq * tile pairs reaches 2^30 or
 *   256 * stride token rows of Q span 4 GiB.  bf16 runs on the matrix
 *   cores; f32 (small problems) forms each sample with f32 dot products. */
int stem_score_antidiag(const stem_plan_info *info, const void *plan_dev,
                        const void *q, const void *k, const float *vnorm, int32_t stride,
                        float *scores, void *stream);

/* stem_select - Token Position-Decay top-k (gist.science/es
 * "Implementacion" steps 2-3, gist.science/nl "Implementatie" steps 2-3).
 * For each (query head, query block i): the sinks {0 .. min(S, i+1) - 1}
 * and the diagonal i are forced; of the candidates {S .. i-1} the
 * k_i - |forced| with the largest metric are kept (equal metric values go
 * to the smaller block number, NaN ranks last).
 *   idx   int32 [Hq, nbT, kmax]: kept local block numbers, ascending, -1 padded
 *   count int32 [Hq, nbT]      : k_i */
int stem_select(const stem_plan_info *info, const void *plan_dev,
                const float *scores, int32_t *idx, int32_t *count,
                void *stream);

/* stem_sparse_attn - exact softmax attention over the kept blocks only
 * (gist.science/es "Implementacion" step 3, gist.science/fr 2.C step 3).
 * Every token t of query block i of head h attends to the tokens of the
 * blocks listed in idx[h, i] (count[h, i] entries, ascending, local block
 * numbers), with key position <= query position (so only the diagonal
 * block is masked inside):
 *   o_t = sum_s softmax_s(q_t . k_s / sqrt(d)) v_s
 * out is [T, Hq, d] in out_dtype (STEM_F32 or STEM_BF16); lse, if not
 * NULL, is f32 [Hq, T] holding the natural-log sum of exp of the scaled
 * logits of each query token.  Listed blocks must lie in [0, i], in
 * ascending order (an entry outside that range, or a list out of order,
 * leads to no access outside the sequence, but the result is not defined),
 * and every row must list at least one block
 * (stem_select always keeps the diagonal block; a row with count 0 has no
 * defined output). */
int stem_sparse_attn(const stem_plan_info *info, const void *plan_dev,
                     const void *q, const void *k, const void *v,
                     const int32_t *idx, const int32_t *count,
                     void *out, int32_t out_dtype, float *lse, void *stream);

/* Measurement probes (not part of the prefill path): they re-measure, on the
 * device at hand, the ceilings the kernels above are compared with.  Each
 * launches one kernel on `stream` and returns at once; the caller times the
 * launch (HIP events on the same stream).  They allocate nothing.
 *
 * stem_probe_mfma - back-to-back bf16 v_mfma_f32_32x32x16 on every SIMD of
 * the current device, four independent accumulators per wavefront.  With
 * random_operands != 0 the operands are random bf16 values in [-1, 1),
 * rotating among four sets, else small constants: the matrix-core rate
 * depends on the operand bit activity (the chip's power limit).  *flops
 * receives the multiply-add work of the launch (2 per multiply-add).  sink
 * is device memory of at least sink_floats f32 (256 x 16 suffice up to 256
 * CUs), overwritten with a value per workgroup.  STEM_EINVAL if a pointer is
 * NULL or sink_floats is smaller than the launch's workgroup count. */
int stem_probe_mfma(int32_t random_operands, float *sink, int64_t sink_floats,
                    double *flops, void *stream);

/* stem_probe_hbm_read - one pass of 16-byte non-temporal loads over the
 * `bytes` bytes at buf (device memory, 16-byte aligned, bytes a positive
 * multiple of 16), the access pattern of the pooling kernel, each workgroup
 * reading one contiguous 64 KiB chunk.  sink is device memory of at least
 * sink_words uint32, sink_words >= ceil(bytes / 65536): word c receives the
 * XOR of the 32-bit words of chunk c, so the XOR of those sink words equals
 * the XOR of the buffer's words.  STEM_EINVAL on a NULL pointer, a bad size,
 * a short sink or misalignment. */
int stem_probe_hbm_read(const void *buf, int64_t bytes, uint32_t *sink, int64_t sink_words,
                        void *stream);

/* Human-readable text of a stem_status value. */
const char *stem_status_str(int status);

#ifdef __cplusplus
}
#endif
#endif /* STEM_H */
