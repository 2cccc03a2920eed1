/*
 * sas.h -- C ABI of the MI355X (gfx950) library for SAS gated block-sparse
 * attention ("SAS: Simple Attention Sparsification via End-to-End
 * Optimization of Context Ranking", arXiv 2609.13141).
 *
 * Pages cited, by title: "review" is the page titled "SAS: Simple Attention
 * Sparsification via End-to-End Optimization of Context Ranking Review"
 * (sections as numbered there); "paper text" is the page titled "SAS: Simple
 * Attention Sparsification via End-to-End Optimization of Context Ranking"
 * that holds the paper's own text (sections 3 and 4, ablation setup and
 * results).
 *
 * The method (as the pages on it describe it):
 *   - a selector scores every history block of 64 tokens; the scores are
 *     turned into gates by a softmax over the history blocks while the
 *     always-kept current block keeps gate 1 (review, section 2-1:
 *     g = phi(s) with g0 = 1, and 3-3; paper text, section 4);
 *   - a hard Top-K keeps the budgeted history blocks (review section 1-2);
 *   - attention runs on the kept blocks only, with log(gate) added to every
 *     logit of the block: o = softmax(q K_S^T + log g_S) V_S (review
 *     section 2-2; block-sparse form: paper text section 3);
 *   - the backward returns dQ/dK/dV and the per-block log-gate gradient,
 *     through which the language-model loss reaches the selector (review
 *     section 3-6; paper text, ablation results);
 *   - decode scores cached block summaries, takes the Top-K per query group,
 *     and attends to the kept blocks of a (paged) KV cache (review 3-7).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers unless the name ends in _host.
 *     The caller owns all memory; the library never allocates, frees or
 *     synchronises.  Every call is asynchronous on `stream` (a hipStream_t,
 *     NULL = the default stream); pointers must stay valid until the stream
 *     reaches the work.  A call only launches kernels on `stream` (no copy,
 *     fill or memset), so calls can be captured into a HIP graph and
 *     replayed; a replay redoes the same work on the same buffers.
 *   - Arguments are checked on the host before anything is launched.  On a
 *     failed check nothing is launched, no output is touched and a negative
 *     sas_status is returned; sas_last_error() then describes the failure
 *     (thread-local).  A launch failure returns SAS_ERR_HIP.
 *   - Contents of device arrays (selection indices, page ids, sequence
 *     lengths) are not re-checked against their host copies; indices out of
 *     range are skipped by the kernels, NaN inputs give unspecified values.
 *   - Layouts are row-major and contiguous; tensors must be 16-byte aligned.
 *     block = 64 tokens; head_dim in {64, 128}; hq a multiple of hkv, and the
 *     query heads h of one KV head g are h = g*G .. g*G+G-1 (G = hq/hkv);
 *     hq * head_dim at most 2^20 (varlen entry points: SAS_ERR_UNSUPPORTED).
 *   - Varlen ("packed") tensors: tokens of all sequences back to back,
 *     cu_seqlens[s] = first token of sequence s.  Query block i of sequence s
 *     covers tokens [cu_seqlens[s] + 64 i, min(+64, cu_seqlens[s+1])).
 *     A row is one (kv head g, query block): row = g * total_qblocks +
 *     cu_qblocks[s] + i.
 *   - Selections: sel_idx [rows][budget_blocks] int32 holds the kept history
 *     blocks in ascending order, then the current block, then -1 padding;
 *     sel_loggate has the same shape and holds log(gate) per entry
 *     (-inf on padding).
 *   - Results are deterministic: identical inputs give bit-identical outputs.
 */
#ifndef SAS_H_
#define SAS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t sas_status;

#define SAS_OK 0
#define SAS_ERR_NULL (-1)        /* a required pointer is NULL */
#define SAS_ERR_SHAPE (-2)       /* sizes are inconsistent */
#define SAS_ERR_DTYPE (-3)       /* unknown dtype code */
#define SAS_ERR_ALIGN (-4)       /* a tensor is not 16-byte aligned */
#define SAS_ERR_UNSUPPORTED (-5) /* head_dim / block / group size not supported */
#define SAS_ERR_WORKSPACE (-6)   /* workspace missing or too small */
#define SAS_ERR_HIP (-7)         /* the HIP runtime reported an error */

#define SAS_BF16 0
#define SAS_F32 1

/* Gate activation.  SAS_GATE_HIST is the pages' method: softmax over the
 * history blocks j < i, the current block keeps log gate 0 (review section
 * 2-1, g0 = 1; paper text: the normaliser is not applied to the current
 * block).  SAS_GATE_ALL normalises over j <= i, the current block included.
 * The activation ablations (paper text section 4; review 3-3), the current
 * block unbiased in both: SAS_GATE_SIGMOID gives independent gates
 * g_j = sigmoid(s_j), SAS_GATE_RAW injects the raw logit (log g_j = s_j);
 * they have no normaliser and write gate_lse = 0.  SAS_GATE_STE is the
 * ranking-preservation ablation: hard gates (log g = 0 on every kept block)
 * in the forward, the history softmax's straight-through gradient in the
 * backward; gate_lse is the soft normaliser. */
#define SAS_GATE_HIST 0
#define SAS_GATE_ALL 1
#define SAS_GATE_SIGMOID 2
#define SAS_GATE_RAW 3
#define SAS_GATE_STE 4

/* Gate position (the gate-position ablation: review 3-2; paper text
 * section 4 and ablation results).  SAS_GATE_INNER adds log g to the logits
 * inside the softmax (the method).  SAS_GATE_OUTER takes the softmax of the
 * ungated logits and scales each key's value by its block's gate:
 *   o_t = sum_u softmax_u(scale q_t.k_u) g_blk(u) v_u,
 * lse is then that of the ungated logits, and d_loggate of a kept block is
 * the sum over its keys of P dP with dP_tu = g (dO_t . v_u). */
#define SAS_GATE_INNER 0
#define SAS_GATE_OUTER 1

#define SAS_KV_CONTIGUOUS 0 /* cache [batch][hkv][max_seqlen][head_dim] */
#define SAS_KV_PAGED 1      /* cache [num_pages][hkv][64][head_dim] + page table */

/* A packed variable-length training / prefill problem. */
typedef struct sas_problem {
  int32_t num_seqs;
  int32_t total_tokens;    /* T = cu_seqlens[num_seqs] */
  int32_t total_qblocks;   /* QB = sum over sequences of ceil(len / 64) */
  int32_t hq, hkv;         /* query heads, key/value heads */
  int32_t head_dim;        /* 64 or 128 */
  int32_t block;           /* 64 */
  int32_t budget_blocks;   /* Kb: kept blocks per row, current block included */
  int32_t dtype;           /* q, k, v: SAS_BF16 or SAS_F32 */
  int32_t out_dtype;       /* o (and dO in sas_bwd): SAS_BF16 or SAS_F32 */
  float scale;             /* softmax scale on q.k (the gate is not scaled) */
  const int32_t *cu_seqlens;       /* device [num_seqs + 1] */
  const int32_t *cu_qblocks;       /* device [num_seqs + 1] */
  const int32_t *cu_seqlens_host;  /* host copies of the two arrays above */
  const int32_t *cu_qblocks_host;
  int32_t gate_position;   /* SAS_GATE_INNER (0, the method) or SAS_GATE_OUTER */
} sas_problem;

/* A single-token decode problem over a KV cache. */
/* Block-summary storage (the pages name reduced-precision summaries as the
 * way to cut the selector scan's bytes): SAS_SUMMARY_BF16 stores each fp32
 * mean rounded to the nearest bf16 (ties to even), and the pooled score
 * reads those rounded values; the score arithmetic is unchanged. */
#define SAS_SUMMARY_F32 0
#define SAS_SUMMARY_BF16 1
/* fp8 e4m3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities; the two codes with exponent and mantissa all ones are NaN):
 * each fp32 mean rounded to the nearest e4m3 value, ties to even; values
 * of 480 or more become NaN.  One byte per value, a quarter of fp32. */
#define SAS_SUMMARY_FP8 2

typedef struct sas_decode_problem {
  int32_t batch;
  int32_t hq, hkv, head_dim, block, budget_blocks;
  int32_t dtype;           /* q and caches: SAS_BF16 */
  int32_t out_dtype;       /* o: SAS_BF16 or SAS_F32 */
  int32_t layout;          /* SAS_KV_CONTIGUOUS or SAS_KV_PAGED */
  int32_t max_seqlen;      /* contiguous: cache capacity per (batch, kv head) */
  int32_t max_pages;       /* paged: row stride of page_table */
  int32_t num_pages;       /* paged: physical pages in the cache */
  int32_t nblk_stride;     /* summaries and scores: blocks per row, a multiple
                              of 64 (>= largest history count) */
  float scale;
  const int32_t *seqlens;       /* device [batch]: cache length L, query token included */
  const int32_t *seqlens_host;  /* host copy */
  const int32_t *page_table;    /* device [batch][max_pages] (paged only) */
  int32_t summary_dtype;        /* block summaries: SAS_SUMMARY_F32, _BF16 or _FP8 */
  const int32_t *page_table_host; /* optional host copy of page_table (paged only): when
                                     given, every entry a sequence uses (its first
                                     ceil(L_b / 64)) is checked to lie in [0, num_pages)
                                     before any launch (SAS_ERR_SHAPE otherwise); when
                                     NULL the device entries are trusted */
  int32_t num_splits;           /* sas_decode: 0 = the library picks the split of every
                                   row's kept blocks over workgroups (enough workgroups
                                   to fill the device's compute units); n >= 1 asks for
                                   n splits (at most budget_blocks; fewer when n does
                                   not divide the blocks evenly).  The split changes
                                   only the fp32 summation order of the result. */
} sas_decode_problem;

/*
 * sas_gate_topk -- gate + hard Top-K for every training row (review 1-2,
 * 2-1, 3-3; paper text section 4).
 *   logits      [hkv][total_qblocks][ld] fp32: column j = key block j of the
 *               row's own sequence; only columns j < i (and j = i in
 *               SAS_GATE_ALL) are read.  ld >= the longest sequence's blocks.
 *   gate_mode   SAS_GATE_HIST, SAS_GATE_ALL, SAS_GATE_SIGMOID, SAS_GATE_RAW
 *               or SAS_GATE_STE.
 *   sel_idx     out [rows][Kb] int32; sel_loggate out [rows][Kb] fp32;
 *   gate_lse    out [rows] fp32: log of the gate normaliser (-inf when empty).
 * Top-K compares the stored fp32 logits: larger first, lower index on ties,
 * -0 equal to +0.  k = min(Kb - 1, i) history blocks are kept.
 */
sas_status sas_gate_topk(const sas_problem *p, const float *logits, int64_t ld,
                         int32_t gate_mode, int32_t *sel_idx, float *sel_loggate,
                         float *gate_lse, void *stream);

/*
 * sas_fwd -- gated block-sparse attention forward (review 2-2, 3-6).
 *   q [T][hq][d], k/v [T][hkv][d] in p->dtype; o [T][hq][d] in p->out_dtype;
 *   lse out [hq][T] fp32, natural-log row log-sum-exp of the gated logits.
 * Token t of query block i attends the kept history blocks whole and the
 * keys u <= t of block i; logit = scale * q.k + sel_loggate of the block.
 */
sas_status sas_fwd(const sas_problem *p, const void *q, const void *k, const void *v,
                   const int32_t *sel_idx, const float *sel_loggate, void *o, float *lse,
                   void *stream);

/*
 * sas_bwd -- gradients of sas_fwd (review 3-6; paper text, ablation results).
 *   o and dO in p->out_dtype; lse from sas_fwd.
 *   dq [T][hq][d], dk/dv [T][hkv][d], d_loggate [rows][Kb]: fp32 outputs,
 *   overwritten (d_loggate padding slots are 0).  d_loggate holds
 *   sum over the row's tokens, its G heads and the block's keys of
 *   dS = P (dP - D), the gradient of the loss with respect to log(gate).
 *   workspace: device scratch of at least sas_bwd_workspace_size(p) bytes.
 */
size_t sas_bwd_workspace_size(const sas_problem *p);
sas_status sas_bwd(const sas_problem *p, const void *q, const void *k, const void *v,
                   const void *o, const void *dO, const float *lse, const int32_t *sel_idx,
                   const float *sel_loggate, float *dq, float *dk, float *dv,
                   float *d_loggate, void *workspace, size_t workspace_bytes, void *stream);

/*
 * The three phases sas_bwd runs, in this order on one workspace (a caller
 * may time them or place them on its own streams, keeping the order):
 *   sas_bwd_prepare  lists, for every (kv head, key block), the (query
 *                    block, slot) pairs that keep it, in query-block order.
 *   sas_bwd_dq       dq and d_loggate; also stores in the workspace the
 *                    exact row term D_t = sum_u P_tu dP_tu that dk needs.
 *   sas_bwd_dkdv     dk and dv; reads the lists and D_t written above.
 * budget_blocks is limited by LDS in sas_bwd_dq (SAS_ERR_UNSUPPORTED when
 * it does not fit: at most about 100 blocks at head_dim 128 in bf16).
 */
sas_status sas_bwd_prepare(const sas_problem *p, const int32_t *sel_idx, void *workspace,
                           size_t workspace_bytes, void *stream);
sas_status sas_bwd_dq(const sas_problem *p, const void *q, const void *k, const void *v,
                      const void *o, const void *dO, const float *lse, const int32_t *sel_idx,
                      const float *sel_loggate, float *dq, float *d_loggate, void *workspace,
                      size_t workspace_bytes, void *stream);
sas_status sas_bwd_dkdv(const sas_problem *p, const void *q, const void *k, const void *v,
                        const void *dO, const float *lse, const float *sel_loggate, float *dk,
                        float *dv, void *workspace, size_t workspace_bytes, void *stream);

/*
 * sas_gate_bwd -- selector-logit gradient from the log-gate gradient through
 * the gate softmax (review 2-1; paper text, ablation results: the normaliser
 * is shared by all history blocks):
 *   d s_m = [m kept] dlg_m - exp(s_m - gate_lse) * sum over kept j of dlg_j
 * for m in the normaliser set; other columns (up to ld) are written 0.
 * In SAS_GATE_HIST the current block's slot carries no gradient.  With
 * independent gates only kept history blocks get one:
 *   SAS_GATE_SIGMOID  d s_m = [m kept] dlg_m * sigmoid(-s_m)
 *   SAS_GATE_RAW      d s_m = [m kept] dlg_m   (gate_lse is not read)
 * and straight-through, with g = exp(s - gate_lse) the soft history gates:
 *   SAS_GATE_STE      d s_m = g_m ([m kept] dlg_m - sum over kept j of g_j dlg_j)
 *   d_logits out [hkv][total_qblocks][ld] fp32.
 */
sas_status sas_gate_bwd(const sas_problem *p, const float *logits, int64_t ld,
                        int32_t gate_mode, const int32_t *sel_idx, const float *gate_lse,
                        const float *d_loggate, float *d_logits, void *stream);

/*
 * sas_pool_keys -- cached block summaries for decode (review 3-7 step 1):
 * the mean key of each full history block j < (L_b - 1) / 64, summed in
 * token order in fp32 and divided by 64.
 *   k_cache in p->layout; ksum out in p->summary_dtype (fp32, or the fp32 mean rounded to
 *   the nearest bf16 / e4m3 value, ties to even), in tiles of 64 blocks:
 *   element [b][g][j / 64][e / EPP][j % 64][e % EPP] is channel e of block j,
 *   EPP = 16 / element size (4, 8 or 16 channels per 16 bytes), so the
 *   16-byte pieces of 64 consecutive blocks lie side by side.
 */
sas_status sas_pool_keys(const sas_decode_problem *p, const void *k_cache, void *ksum,
                         void *stream);

/*
 * sas_decode_append -- one decode step's cache maintenance (review 3-7: the
 * block summaries follow the growing cache).  p->seqlens already count the
 * new token (L_b), which is written at position L_b - 1 of every kv head's
 * row; when that position opens a new block (L_b - 1 a positive multiple
 * of 64), the block before it has become history and its summary is
 * written, with exactly the value sas_pool_keys gives it.  Together with
 * sas_pool_keys over a prefilled prefix (the dense-prefill handoff) this
 * keeps ksum equal to sas_pool_keys of the whole cache after every step.
 *   k_new, v_new  [batch][hkv][head_dim] bf16 (the new token's key, value);
 *   k_cache, v_cache in p->layout (updated in place; paged: the page of
 *                 position L_b - 1 must be in the page table); ksum
 *                 (the tiled layout of sas_pool_keys) in p->summary_dtype,
 *                 updated in place.
 * The caller owns every buffer; NULL -> SAS_ERR_NULL, bad shapes as for
 * sas_pool_keys.  Steps are ordered on the stream; the summary read uses
 * tokens written by earlier steps only.
 *   csum: the super-block summaries of the hierarchical selection
 *         (sas_pool_coarse), or NULL when they are not kept; when the
 *         summary written completes a super-block (its index + 1 a multiple
 *         of SAS_COARSE_BLOCKS), that super-block's summary is written too,
 *         with exactly the value sas_pool_coarse gives it.
 */
sas_status sas_decode_append(const sas_decode_problem *p, const void *k_new, const void *v_new,
                             void *k_cache, void *v_cache, void *ksum, void *csum,
                             void *stream);

/*
 * sas_decode_select -- decode-time selection (review 3-7 steps 1-2; GQA
 * groups share one selection; review 4-4 and 6: the scan over every cached
 * block is what limits long contexts): per (batch b, kv head g) row,
 *   qbar_e = (q_{gG} + ... + q_{gG+G-1})_e / G   (fp32, heads in order)
 *   s_j    = (fmaf chain over e of qbar_e * ksum_je) / sqrtf(head_dim)
 * then the gate + Top-K of sas_gate_topk with i = (L_b - 1) / 64 and
 * SAS_GATE_HIST.  q [batch][hq][d] bf16; ksum in the tiled layout of
 * sas_pool_keys, p->summary_dtype, 16-byte aligned.
 *   sel_idx / sel_loggate out [batch*hkv][Kb]; gate_lse out [batch*hkv];
 *   scores out [batch][hkv][nblk_stride] fp32 (the pooled scores).
 * Each row's history is split into chunks taken by separate workgroups
 * (scores and an exact Top-K per chunk), merged per row by a second kernel;
 * the result is the whole row's Top-K.
 *   workspace: at least sas_decode_select_workspace_size(p) bytes (any
 *   contents; calls that share a workspace must not overlap in time).
 * A row's history is split into chunks of 256 to 2048 blocks (512 for a
 * many-row batch with bf16 or fp8 summaries); more than
 * 4096 candidates in the merge (chunks x (Kb - 1)) returns
 * SAS_ERR_UNSUPPORTED (at Kb = 32: histories beyond 270,336 blocks, 17M
 * tokens).
 */
size_t sas_decode_select_workspace_size(const sas_decode_problem *p);
sas_status sas_decode_select(const sas_decode_problem *p, const void *q, const void *ksum,
                             float *scores, int32_t *sel_idx, float *sel_loggate,
                             float *gate_lse, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * Hierarchical (coarse-to-fine) selection (review 7-2: a coarse retrieval
 * narrows the candidate blocks, then the selector picks its Top-K among
 * them, so the scan reads far fewer summaries on long contexts).  An
 * approximation of sas_decode_select, opt-in: it equals sas_decode_select
 * whenever every super-block is kept.
 *
 * A super-block is SAS_COARSE_BLOCKS consecutive history blocks; only
 * complete super-blocks (all their blocks history) have a summary.
 *
 * sas_pool_coarse -- super-block summaries from the block summaries: the
 * mean of the SAS_COARSE_BLOCKS stored block summaries (their fp32 values,
 * summed in block order in fp32, divided by SAS_COARSE_BLOCKS), stored in
 * p->summary_dtype like them.  ksum as written by sas_pool_keys; csum out
 * in the same tiled layout with cstride = ceil(nblk_stride /
 * SAS_COARSE_BLOCKS / 64) * 64 super-blocks per row:
 * [batch][hkv][cstride / 64][head_dim / EPP][64][EPP].
 */
#define SAS_COARSE_BLOCKS 8
sas_status sas_pool_coarse(const sas_decode_problem *p, const void *ksum, void *csum,
                           void *stream);

/*
 * sas_decode_select_hier -- per (batch b, kv head g) row: the pooled score
 * of every super-block summary (the fmaf chain of sas_decode_select); the
 * coarse_keep best super-blocks (earlier on ties); the candidates are all
 * blocks of those super-blocks and the trailing history blocks that form no
 * complete super-block, in block order; then the gate and Top-K of
 * sas_decode_select over the candidates only (the normaliser gate_lse runs
 * over the candidates).  Outputs as sas_decode_select; scores are written
 * for the candidate blocks only.  1 <= coarse_keep <= 127 (SAS_ERR_SHAPE
 * otherwise).  Three launches (coarse chunks, coarse merge, fine pass).
 *   workspace: at least sas_decode_select_hier_workspace_size(p, coarse_keep)
 *   bytes (any contents; calls sharing one must not overlap in time).
 */
size_t sas_decode_select_hier_workspace_size(const sas_decode_problem *p, int32_t coarse_keep);
sas_status sas_decode_select_hier(const sas_decode_problem *p, const void *q, const void *ksum,
                                  const void *csum, int32_t coarse_keep, float *scores,
                                  int32_t *sel_idx, float *sel_loggate, float *gate_lse,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * sas_decode -- block-sparse decode attention (review 3-7 steps 3-4) for
 * the newest token of every sequence: each of the G query heads of (b, g)
 * attends the kept history blocks and the present tokens of the current
 * block, log gates added per block (sel_loggate NULL: no gate).  Work is
 * split over kept blocks and merged with a log-sum-exp combine.
 *   q [batch][hq][d] bf16; o out [batch][hq][d] in p->out_dtype;
 *   lse out [batch][hq] fp32 or NULL.
 *   workspace: at least sas_decode_workspace_size(p) bytes.
 */
/* The workspace size depends only on the problem (for num_splits = 0 it is
 * sized for the largest split the library may pick on any device). */
size_t sas_decode_workspace_size(const sas_decode_problem *p);
sas_status sas_decode(const sas_decode_problem *p, const void *q, const void *k_cache,
                      const void *v_cache, const int32_t *sel_idx, const float *sel_loggate,
                      void *o, float *lse, void *workspace, size_t workspace_bytes,
                      void *stream);

/*
 * sas_decode_noalloc -- sas_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments and results as sas_decode, without
 * the workspace: the split partials go to a fixed scratch array inside the
 * library, SAS_DECODE_SCRATCH_BYTES per device, held by each device that
 * runs the library until the process ends.  It allocates nothing (no
 * hipMalloc / hipFree, no allocating library routine).
 *   A problem whose partials, batch * hkv * splits * G * (head_dim + 2)
 *   floats, exceed the scratch returns SAS_ERR_WORKSPACE before any launch
 *   (rows split once need no scratch).
 *   Every call on one device shares that device's scratch: calls on one
 *   stream are ordered, calls that overlap in time on one device (other
 *   streams, other threads) race and must not be issued.
 */
#define SAS_DECODE_SCRATCH_BYTES (4u << 20)
sas_status sas_decode_noalloc(const sas_decode_problem *p, const void *q, const void *k_cache,
                              const void *v_cache, const int32_t *sel_idx,
                              const float *sel_loggate, void *o, float *lse, void *stream);

/* Static description of a status code. */
const char *sas_status_string(sas_status s);
/* Detail of the last failed call on this thread ("" if none). */
const char *sas_last_error(void);
/* ABI version of this header: bumped on any incompatible change. */
int32_t sas_abi_version(void);

#define SAS_ABI_VERSION 6

#ifdef __cplusplus
}
#endif

#endif /* SAS_H_ */
