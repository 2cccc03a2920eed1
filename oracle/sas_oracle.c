/*
 * SAS gated block-sparse attention -- plain CPU oracle, fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: it exists so that tests, the smoke check and the CPU
 * baseline leg of the benchmark can check the HIP library against a slow,
 * obviously correct restatement of the method.  It shares no code, header,
 * table or constant with the HIP library.
 *
 * Sources (the pages on "SAS: Simple Attention Sparsification via End-to-End
 * Optimization of Context Ranking", arXiv 2609.13141), cited by title:
 *   [R]  the page titled "SAS: Simple Attention Sparsification via End-to-End
 *        Optimization of Context Ranking Review", sections: 1-1 (dense and block-sparse attention
 *        equations), 1-2 (hard Top-K equation), 2-1 (g = phi(s), g0 = 1,
 *        broadcast), 2-2 (inner log-gate equation and the softmax/log identity),
 *        3-3 (softmax gate activation), 3-5 (sparse scope), 3-6 (fused kernel,
 *        backward keeps the selector gradient), 3-7 (decode path steps 1-4),
 *        7-2 (a coarse retrieval narrowing the candidates before the Top-K).
 *   [P]  the page titled "SAS: Simple Attention Sparsification via End-to-End
 *        Optimization of Context Ranking" holding the paper's own text: section 3 (standard attention,
 *        scaling factor omitted, block partition, Top-K selected index set),
 *        section 4 (current block singled out and unbiased, gate broadcast,
 *        gate-position/activation/scope design elements), ablation results
 *        (the inner gate's gradient measures a block against the row's
 *        mean, the normaliser is shared by the
 *        historical blocks and not applied to the current block, invariance
 *        to a global shift of the scores).
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - logits are z = scale * q.k + log g; the gate itself is not scaled.
 *   - GATE_HIST (mode 0, the pages' reading): g = softmax over the history
 *     blocks j < i only, the current block keeps log g = 0.
 *     GATE_ALL (mode 1): softmax over j <= i, current block included.
 *     The activation ablations of [P] section 4 / [R] 3-3, with the current
 *     block unbiased in both: GATE_SIGMOID (mode 2): independent gates
 *     g_j = sigmoid(s_j), log g_j = -log(1 + exp(-s_j)); GATE_RAW (mode 3):
 *     the unnormalised logit injected as is, log g_j = s_j.  These have no
 *     normaliser; their gate_lse output is 0.
 *     GATE_STE (mode 4), the ranking-preservation ablation: a hard gate
 *     (log g = 0, gate 1, on every kept block) in the forward, with the
 *     straight-through gradient of the soft history softmax in the backward:
 *     the loss gradient with respect to a kept block's gate is taken as the
 *     gradient with respect to its soft gate g_j = exp(s_j - lse), so
 *       d s_m = sum over kept j of dL/dg_j * g_j ([j = m] - g_m)
 *     with dL/dg_j = d log g_j (the hard gate is 1).  gate_lse is the soft
 *     normaliser.
 *   - the normaliser runs over every causal history candidate; the Top-K then
 *     keeps a subset, so kept gates sum to at most 1.
 *   - budget Kb counts the current block; k = min(Kb - 1, i) history blocks.
 *   - Top-K on the stored fp32 logits, larger first, lower index on ties
 *     (-0 and +0 compare equal).
 *   - a token attends to keys u <= t inside its own block (self included).
 *   - all-(-inf) normaliser sets give log g = -inf (gate 0).
 *   - decode: cache length L counts the query's own token; the current block
 *     is cur = (L-1)/b and may be partial; block summaries exist for j < cur.
 *   - decode scores are computed in fp32 in one fixed order so that both
 *     sides take the Top-K decision on identical values:
 *       kbar[j][e] = (((k0 + k1) + k2) + ... + k63) / 64        (fp32, in order)
 *       qbar[e]    = (((q0 + q1) + ... + q_{G-1})) / G          (fp32, in order)
 *       A          = fmaf(qbar[e], kbar[j][e], A)  for e = 0..d-1 (fp32)
 *       s_j        = A / sqrtf(d)                                (fp32)
 *   - hierarchical selection (opt-in): super-blocks of F = 8 history blocks;
 *     a complete super-block's summary is the mean of its F stored block
 *     summaries (summed in block order in fp32, divided by F, rounded like
 *     them); the best super-blocks by the same pooled score (earlier on
 *     ties) and the trailing blocks of no complete super-block are the
 *     candidates, and the gate and Top-K run over the candidates only.
 *
 * Layouts (all row-major, C order):
 *   q, o, dq        [T][hq][d]        k, v, dk, dv   [T][hkv][d]
 *   lse             [hq][T]           logits         [hkv][QB][ld]
 *   sel_idx, sel_lg, dlg              [hkv][QB][Kb]  gate_lse [hkv][QB]
 * where T = cu_seqlens[nseq], QB = sum over sequences of ceil(len / b), and a
 * row r = g * QB + (first query block of the sequence) + i.
 * sel_idx of a row: the kept history blocks ascending, then the current
 * block i, then -1 padding (with log gate -inf).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_GATE_HIST 0
#define ORACLE_GATE_ALL 1
#define ORACLE_GATE_SIGMOID 2
#define ORACLE_GATE_RAW 3
#define ORACLE_GATE_STE 4

/* log sigmoid(x) = -log(1 + exp(-x)), written so that neither branch
 * overflows: for x < 0 it is x - log(1 + exp(x)). */
static double log_sigmoid(double x) {
  if (x >= 0.0) return -log1p(exp(-x));
  return x - log1p(exp(x));
}

static int ceil_div(int a, int b) { return (a + b - 1) / b; }

/* Prefix sums of query blocks per sequence; returns the total. */
static int query_block_offsets(int nseq, const int32_t *cu, int blk, int *cuqb) {
  cuqb[0] = 0;
  for (int s = 0; s < nseq; ++s) cuqb[s + 1] = cuqb[s] + ceil_div(cu[s + 1] - cu[s], blk);
  return cuqb[nseq];
}

static int seq_of_qblock(int nseq, const int *cuqb, int Q) {
  int s = 0;
  while (s + 1 < nseq && cuqb[s + 1] <= Q) ++s;
  return s;
}

int sas_oracle_num_qblocks(int nseq, const int32_t *cu, int blk) {
  int *cuqb = (int *)malloc(sizeof(int) * (nseq + 1));
  int n = query_block_offsets(nseq, cu, blk, cuqb);
  free(cuqb);
  return n;
}

/*
 * One gate row ([R] 2-1 g = phi(s) with g0 = 1, 3-3 softmax activation;
 * [P] section 4 current block unbiased; [R] 1-2 I = TopK(s, K)).
 * s: the row's scores for blocks 0..i (s[i] read only in GATE_ALL mode).
 */
static void gate_row(const float *s, int i, int Kb, int mode, int32_t *idx, double *lg,
                     double *lse_out, unsigned char *chosen) {
  int independent = (mode == ORACLE_GATE_SIGMOID || mode == ORACLE_GATE_RAW);
  int nn = (mode == ORACLE_GATE_ALL) ? i + 1 : i; /* size of the normaliser set */
  double lse = independent ? 0.0 : -INFINITY;
  if (nn > 0 && !independent) {
    double m = -INFINITY;
    for (int j = 0; j < nn; ++j)
      if ((double)s[j] > m) m = (double)s[j];
    if (m != -INFINITY) {
      double acc = 0.0;
      for (int j = 0; j < nn; ++j) acc += exp((double)s[j] - m);
      lse = m + log(acc);
    }
  }
  *lse_out = lse;

  /* Hard Top-K over the history blocks: repeatedly take the largest score,
   * the lowest index winning ties.  Quadratic, which is fine here. */
  int k = Kb - 1 < i ? Kb - 1 : i;
  memset(chosen, 0, (size_t)(i > 0 ? i : 1));
  for (int t = 0; t < k; ++t) {
    int best = -1;
    for (int j = 0; j < i; ++j) {
      if (chosen[j]) continue;
      if (best < 0 || s[j] > s[best]) best = j;
    }
    chosen[best] = 1;
  }
  int pos = 0;
  for (int j = 0; j < i; ++j) {
    if (!chosen[j]) continue;
    idx[pos] = j;
    if (mode == ORACLE_GATE_SIGMOID)
      lg[pos] = log_sigmoid((double)s[j]);
    else if (mode == ORACLE_GATE_RAW)
      lg[pos] = (double)s[j];
    else if (mode == ORACLE_GATE_STE)
      lg[pos] = 0.0; /* hard gate: every kept block weighs 1 */
    else
      lg[pos] = (lse == -INFINITY) ? -INFINITY : (double)s[j] - lse;
    ++pos;
  }
  idx[pos] = i;
  if (mode == ORACLE_GATE_ALL)
    lg[pos] = (lse == -INFINITY) ? -INFINITY : (double)s[i] - lse;
  else
    lg[pos] = 0.0;
  ++pos;
  for (; pos < Kb; ++pos) {
    idx[pos] = -1;
    lg[pos] = -INFINITY;
  }
}

int sas_oracle_gate_topk(int nseq, const int32_t *cu, int blk, int hkv, int Kb, int mode,
                         const float *logits, int64_t ld, int32_t *sel_idx, double *sel_lg,
                         double *gate_lse) {
  if (nseq <= 0 || blk <= 0 || hkv <= 0 || Kb < 1) return -1;
  int *cuqb = (int *)malloc(sizeof(int) * (nseq + 1));
  int QB = query_block_offsets(nseq, cu, blk, cuqb);
  int maxi = 0;
  for (int s = 0; s < nseq; ++s)
    if (cuqb[s + 1] - cuqb[s] > maxi) maxi = cuqb[s + 1] - cuqb[s];
  if (ld < maxi) {
    free(cuqb);
    return -2;
  }
  long nrows = (long)hkv * QB;
#pragma omp parallel
  {
    unsigned char *chosen = (unsigned char *)malloc((size_t)maxi + 1);
#pragma omp for schedule(dynamic, 8)
    for (long r = 0; r < nrows; ++r) {
      int Q = (int)(r % QB);
      int s = seq_of_qblock(nseq, cuqb, Q);
      int i = Q - cuqb[s];
      gate_row(logits + r * ld, i, Kb, mode, sel_idx + r * Kb, sel_lg + r * Kb, gate_lse + r,
               chosen);
    }
    free(chosen);
  }
  free(cuqb);
  return 0;
}

/* Gate + Top-K for one row given its scores directly (decode rows). */
int sas_oracle_gate_row(const float *scores, int i, int Kb, int mode, int32_t *idx, double *lg,
                        double *lse) {
  unsigned char *chosen = (unsigned char *)malloc((size_t)i + 1);
  gate_row(scores, i, Kb, mode, idx, lg, lse, chosen);
  free(chosen);
  return 0;
}

/*
 * The attended key list of one query token ([R] 1-1 block-sparse equation,
 * 2-2 inner log gate, 2-1 broadcast of a block's gate to its tokens;
 * [P] section 3 union of the selected blocks).  Fills u[] (global key rows)
 * and slot[] (index into the row's selection) and returns the count.
 */
static int attended_keys(const int32_t *idx, int Kb, int i, int blk, int seq_start, int seq_len,
                         int t_local, int *u, int *slot) {
  int n = 0;
  for (int sl = 0; sl < Kb; ++sl) {
    int j = idx[sl];
    if (j < 0) continue;
    int lo = j * blk, hi = lo + blk;
    if (hi > seq_len) hi = seq_len;
    if (j == i && hi > t_local + 1) hi = t_local + 1; /* causal inside the current block */
    for (int p = lo; p < hi; ++p) {
      u[n] = seq_start + p;
      slot[n] = sl;
      ++n;
    }
  }
  return n;
}

static double dot_dd(const double *a, const double *b, int d) {
  double acc = 0.0;
  for (int e = 0; e < d; ++e) acc += a[e] * b[e];
  return acc;
}

/*
 * Forward ([R] 2-2: o = softmax(q K_S^T + log g_S) V_S, with the scale the
 * paper text says it omits for brevity restored).  Rows whose row_mask entry
 * is 0 are skipped (row_mask may be NULL: every row).
 */
int sas_oracle_fwd(int nseq, const int32_t *cu, int blk, int hq, int hkv, int d, int Kb,
                   double scale, const double *q, const double *k, const double *v,
                   const int32_t *sel_idx, const double *sel_lg, const unsigned char *row_mask,
                   double *o, double *lse) {
  if (hq % hkv) return -1;
  int G = hq / hkv;
  int *cuqb = (int *)malloc(sizeof(int) * (nseq + 1));
  int QB = query_block_offsets(nseq, cu, blk, cuqb);
  int T = cu[nseq];
  long nrows = (long)hkv * QB;
  int maxkeys = Kb * blk;
#pragma omp parallel
  {
    int *u = (int *)malloc(sizeof(int) * maxkeys);
    int *slot = (int *)malloc(sizeof(int) * maxkeys);
    double *z = (double *)malloc(sizeof(double) * maxkeys);
#pragma omp for schedule(dynamic, 1)
    for (long r = 0; r < nrows; ++r) {
      if (row_mask && !row_mask[r]) continue;
      int g = (int)(r / QB), Q = (int)(r % QB);
      int s = seq_of_qblock(nseq, cuqb, Q);
      int i = Q - cuqb[s];
      int start = cu[s], len = cu[s + 1] - cu[s];
      const int32_t *idx = sel_idx + r * Kb;
      const double *lg = sel_lg + r * Kb;
      for (int tl = i * blk; tl < (i + 1) * blk && tl < len; ++tl) {
        int t = start + tl;
        int n = attended_keys(idx, Kb, i, blk, start, len, tl, u, slot);
        for (int hh = 0; hh < G; ++hh) {
          int h = g * G + hh;
          const double *qt = q + ((long)t * hq + h) * d;
          double m = -INFINITY;
          for (int a = 0; a < n; ++a) {
            z[a] = scale * dot_dd(qt, k + ((long)u[a] * hkv + g) * d, d) + lg[slot[a]];
            if (z[a] > m) m = z[a];
          }
          double den = 0.0;
          for (int a = 0; a < n; ++a) den += exp(z[a] - m);
          double *ot = o + ((long)t * hq + h) * d;
          for (int e = 0; e < d; ++e) ot[e] = 0.0;
          for (int a = 0; a < n; ++a) {
            double p = exp(z[a] - m) / den;
            const double *vu = v + ((long)u[a] * hkv + g) * d;
            for (int e = 0; e < d; ++e) ot[e] += p * vu[e];
          }
          lse[(long)h * T + t] = m + log(den);
        }
      }
    }
    free(u);
    free(slot);
    free(z);
  }
  free(cuqb);
  return 0;
}

/*
 * Backward: the gradients of the forward above with respect to q, k, v and
 * the per-block log gate, written out by the chain rule (the pages state
 * that the backward keeps the selector gradient, [R] 3-6, and describe the
 * inner gate's gradient as P_gated (dP - D), each block measured against
 * the row's mean, [P] ablation results):
 *   P_tu  = softmax_u(z_t)          D_t   = sum_e dO_te o_te
 *   dP_tu = dO_t . v_u              dS_tu = P_tu (dP_tu - D_t)
 *   dq_t  = scale sum_u dS_tu k_u   dk_u  = scale sum_t dS_tu q_t
 *   dv_u  = sum_t P_tu dO_t         dlg_r,slot = sum over the row's tokens,
 *                                    heads and the slot's keys of dS_tu
 * row_mask selects the rows whose dq / dlg are produced; kblk_mask (indexed
 * like rows: [hkv][QB]) selects the key blocks whose dk / dv are produced,
 * accumulated over every row that attends to them.  NULL masks mean all.
 * Every output is overwritten (zero where not produced).
 */
int sas_oracle_bwd(int nseq, const int32_t *cu, int blk, int hq, int hkv, int d, int Kb,
                   double scale, const double *q, const double *k, const double *v,
                   const double *dO, const int32_t *sel_idx, const double *sel_lg,
                   const unsigned char *row_mask, const unsigned char *kblk_mask, double *dq,
                   double *dk, double *dv, double *dlg) {
  if (hq % hkv) return -1;
  int G = hq / hkv;
  int *cuqb = (int *)malloc(sizeof(int) * (nseq + 1));
  int QB = query_block_offsets(nseq, cu, blk, cuqb);
  int T = cu[nseq];
  long nrows = (long)hkv * QB;
  memset(dq, 0, sizeof(double) * (size_t)T * hq * d);
  memset(dk, 0, sizeof(double) * (size_t)T * hkv * d);
  memset(dv, 0, sizeof(double) * (size_t)T * hkv * d);
  memset(dlg, 0, sizeof(double) * (size_t)nrows * Kb);
  /* Rows whose softmax statistics are needed: those asked for, and those
   * that keep a key block whose dk / dv are asked for. */
  unsigned char *need = (unsigned char *)calloc(nrows > 0 ? nrows : 1, 1);
  for (long r = 0; r < nrows; ++r) {
    int g = (int)(r / QB), Q = (int)(r % QB);
    int s = seq_of_qblock(nseq, cuqb, Q);
    need[r] = row_mask ? row_mask[r] : 1;
    for (int sl = 0; sl < Kb && !need[r]; ++sl) {
      int j = sel_idx[r * Kb + sl];
      if (j >= 0 && (!kblk_mask || kblk_mask[(long)g * QB + cuqb[s] + j])) need[r] = 1;
    }
  }
  /* per (token, head): lse_t = log sum_u exp(z_tu) and D_t = dO_t . o_t */
  double *lse_t = (double *)malloc(sizeof(double) * ((size_t)T * hq + 1));
  double *D_t = (double *)malloc(sizeof(double) * ((size_t)T * hq + 1));
  int maxkeys = Kb * blk;

  /* Query side, one row at a time (rows write disjoint dq and dlg). */
#pragma omp parallel
  {
    int *u = (int *)malloc(sizeof(int) * maxkeys);
    int *slot = (int *)malloc(sizeof(int) * maxkeys);
    double *z = (double *)malloc(sizeof(double) * maxkeys);
    double *P = (double *)malloc(sizeof(double) * maxkeys);
    double *ot = (double *)malloc(sizeof(double) * d);
#pragma omp for schedule(dynamic, 1)
    for (long r = 0; r < nrows; ++r) {
      if (!need[r]) continue;
      int g = (int)(r / QB), Q = (int)(r % QB);
      int s = seq_of_qblock(nseq, cuqb, Q);
      int i = Q - cuqb[s];
      int start = cu[s], len = cu[s + 1] - cu[s];
      const int32_t *idx = sel_idx + r * Kb;
      const double *lg = sel_lg + r * Kb;
      int want_row = row_mask ? row_mask[r] : 1;
      for (int tl = i * blk; tl < (i + 1) * blk && tl < len; ++tl) {
        int t = start + tl;
        int n = attended_keys(idx, Kb, i, blk, start, len, tl, u, slot);
        for (int hh = 0; hh < G; ++hh) {
          int h = g * G + hh;
          const double *qt = q + ((long)t * hq + h) * d;
          const double *dOt = dO + ((long)t * hq + h) * d;
          double m = -INFINITY;
          for (int a = 0; a < n; ++a) {
            z[a] = scale * dot_dd(qt, k + ((long)u[a] * hkv + g) * d, d) + lg[slot[a]];
            if (z[a] > m) m = z[a];
          }
          double den = 0.0;
          for (int a = 0; a < n; ++a) den += exp(z[a] - m);
          for (int e = 0; e < d; ++e) ot[e] = 0.0;
          for (int a = 0; a < n; ++a) {
            P[a] = exp(z[a] - m) / den;
            const double *vu = v + ((long)u[a] * hkv + g) * d;
            for (int e = 0; e < d; ++e) ot[e] += P[a] * vu[e];
          }
          double D = 0.0;
          for (int e = 0; e < d; ++e) D += dOt[e] * ot[e];
          lse_t[(long)t * hq + h] = m + log(den);
          D_t[(long)t * hq + h] = D;
          if (!want_row) continue;
          double *dqt = dq + ((long)t * hq + h) * d;
          for (int a = 0; a < n; ++a) {
            const double *ku = k + ((long)u[a] * hkv + g) * d;
            const double *vu = v + ((long)u[a] * hkv + g) * d;
            double dS = P[a] * (dot_dd(dOt, vu, d) - D);
            for (int e = 0; e < d; ++e) dqt[e] += scale * dS * ku[e];
            dlg[r * Kb + slot[a]] += dS;
          }
        }
      }
    }
    free(u);
    free(slot);
    free(z);
    free(P);
    free(ot);
  }

  /* Key side, one key block at a time (blocks write disjoint dk and dv):
   * for key u of block j, the sum over every (row, token, head) that
   * attends to it, in row, token, head order, of
   *   P_tu = exp(z_tu - lse_t),  dS_tu = P_tu (dO_t . v_u - D_t). */
#pragma omp parallel for schedule(dynamic, 1)
  for (long x = 0; x < nrows; ++x) {
    if (kblk_mask && !kblk_mask[x]) continue;
    int g = (int)(x / QB), Qk = (int)(x % QB);
    int s = seq_of_qblock(nseq, cuqb, Qk);
    int j = Qk - cuqb[s];
    int start = cu[s], len = cu[s + 1] - cu[s];
    int nb = cuqb[s + 1] - cuqb[s];
    int lo = j * blk, hi = lo + blk < len ? lo + blk : len;
    for (int i = j; i < nb; ++i) {
      long r = (long)g * QB + cuqb[s] + i;
      int sl = -1;
      for (int c = 0; c < Kb; ++c)
        if (sel_idx[r * Kb + c] == j) sl = c;
      if (sl < 0) continue;
      double lg = sel_lg[r * Kb + sl];
      for (int tl = i * blk; tl < (i + 1) * blk && tl < len; ++tl) {
        int t = start + tl;
        for (int pu = lo; pu < hi; ++pu) {
          if (i == j && pu > tl) break; /* causal inside the current block */
          long uu = start + pu;
          const double *ku = k + (uu * hkv + g) * d;
          const double *vu = v + (uu * hkv + g) * d;
          double *dku = dk + (uu * hkv + g) * d;
          double *dvu = dv + (uu * hkv + g) * d;
          for (int hh = 0; hh < G; ++hh) {
            int h = g * G + hh;
            const double *qt = q + ((long)t * hq + h) * d;
            const double *dOt = dO + ((long)t * hq + h) * d;
            double z = scale * dot_dd(qt, ku, d) + lg;
            double Ptu = exp(z - lse_t[(long)t * hq + h]);
            double dS = Ptu * (dot_dd(dOt, vu, d) - D_t[(long)t * hq + h]);
            for (int e = 0; e < d; ++e) {
              dku[e] += scale * dS * qt[e];
              dvu[e] += Ptu * dOt[e];
            }
          }
        }
      }
    }
  }
  free(lse_t);
  free(D_t);
  free(need);
  free(cuqb);
  return 0;
}

/*
 * The gate-position ablation ([R] 3-2 outer-gate equation; [P] section 4,
 * "gate position", and the ablation results: outside the softmax the
 * probabilities are fixed and the gate only rescales the value
 * contribution of its block):
 *   o_t = sum_u softmax_u(scale q_t.k_u) g_blk(u) v_u,   g = exp(log g)
 * lse is the row log-sum-exp of the ungated logits.  Backward, by the chain
 * rule, with P the ungated probabilities:
 *   dP_tu = g_blk(u) (dO_t . v_u)    D_t = dO_t . o_t = sum_u P_tu dP_tu
 *   dS_tu = P_tu (dP_tu - D_t)       dq, dk from dS as in the inner gate
 *   dv_u  = sum_t P_tu g_blk(u) dO_t
 *   dlg_r,slot = d L / d log g = sum over the row's tokens, heads and the
 *                slot's keys of P_tu dP_tu   (no -D term: P does not
 *                depend on the gate)
 */
int sas_oracle_fwd_outer(int nseq, const int32_t *cu, int blk, int hq, int hkv, int d, int Kb,
                         double scale, const double *q, const double *k, const double *v,
                         const int32_t *sel_idx, const double *sel_lg, double *o, double *lse) {
  if (hq % hkv) return -1;
  int G = hq / hkv;
  int *cuqb = (int *)malloc(sizeof(int) * (nseq + 1));
  int QB = query_block_offsets(nseq, cu, blk, cuqb);
  int T = cu[nseq];
  long nrows = (long)hkv * QB;
  int maxkeys = Kb * blk;
#pragma omp parallel
  {
    int *u = (int *)malloc(sizeof(int) * maxkeys);
    int *slot = (int *)malloc(sizeof(int) * maxkeys);
    double *z = (double *)malloc(sizeof(double) * maxkeys);
#pragma omp for schedule(dynamic, 1)
    for (long r = 0; r < nrows; ++r) {
      int g = (int)(r / QB), Q = (int)(r % QB);
      int s = seq_of_qblock(nseq, cuqb, Q);
      int i = Q - cuqb[s];
      int start = cu[s], len = cu[s + 1] - cu[s];
      const int32_t *idx = sel_idx + r * Kb;
      const double *lg = sel_lg + r * Kb;
      for (int tl = i * blk; tl < (i + 1) * blk && tl < len; ++tl) {
        int t = start + tl;
        int n = attended_keys(idx, Kb, i, blk, start, len, tl, u, slot);
        for (int hh = 0; hh < G; ++hh) {
          int h = g * G + hh;
          const double *qt = q + ((long)t * hq + h) * d;
          double m = -INFINITY;
          for (int a = 0; a < n; ++a) {
            z[a] = scale * dot_dd(qt, k + ((long)u[a] * hkv + g) * d, d); /* no gate */
            if (z[a] > m) m = z[a];
          }
          double den = 0.0;
          for (int a = 0; a < n; ++a) den += exp(z[a] - m);
          double *ot = o + ((long)t * hq + h) * d;
          for (int e = 0; e < d; ++e) ot[e] = 0.0;
          for (int a = 0; a < n; ++a) {
            double p = exp(z[a] - m) / den;
            double gate = exp(lg[slot[a]]);
            const double *vu = v + ((long)u[a] * hkv + g) * d;
            for (int e = 0; e < d; ++e) ot[e] += p * gate * vu[e];
          }
          lse[(long)h * T + t] = m + log(den);
        }
      }
    }
    free(u);
    free(slot);
    free(z);
  }
  free(cuqb);
  return 0;
}

int sas_oracle_bwd_outer(int nseq, const int32_t *cu, int blk, int hq, int hkv, int d, int Kb,
                         double scale, const double *q, const double *k, const double *v,
                         const double *dO, const int32_t *sel_idx, const double *sel_lg,
                         double *dq, double *dk, double *dv, double *dlg) {
  if (hq % hkv) return -1;
  int G = hq / hkv;
  int *cuqb = (int *)malloc(sizeof(int) * (nseq + 1));
  int QB = query_block_offsets(nseq, cu, blk, cuqb);
  int T = cu[nseq];
  memset(dq, 0, sizeof(double) * (size_t)T * hq * d);
  memset(dk, 0, sizeof(double) * (size_t)T * hkv * d);
  memset(dv, 0, sizeof(double) * (size_t)T * hkv * d);
  memset(dlg, 0, sizeof(double) * (size_t)hkv * QB * Kb);
  int maxkeys = Kb * blk;
  long npairs = (long)hkv * nseq;
#pragma omp parallel
  {
    int *u = (int *)malloc(sizeof(int) * maxkeys);
    int *slot = (int *)malloc(sizeof(int) * maxkeys);
    double *z = (double *)malloc(sizeof(double) * maxkeys);
    double *P = (double *)malloc(sizeof(double) * maxkeys);
    double *ot = (double *)malloc(sizeof(double) * d);
#pragma omp for schedule(dynamic, 1)
    for (long pr = 0; pr < npairs; ++pr) {
      int g = (int)(pr / nseq), s = (int)(pr % nseq);
      int start = cu[s], len = cu[s + 1] - cu[s];
      int nb = cuqb[s + 1] - cuqb[s];
      for (int i = 0; i < nb; ++i) {
        long r = (long)g * QB + cuqb[s] + i;
        const int32_t *idx = sel_idx + r * Kb;
        const double *lg = sel_lg + r * Kb;
        for (int tl = i * blk; tl < (i + 1) * blk && tl < len; ++tl) {
          int t = start + tl;
          int n = attended_keys(idx, Kb, i, blk, start, len, tl, u, slot);
          for (int hh = 0; hh < G; ++hh) {
            int h = g * G + hh;
            const double *qt = q + ((long)t * hq + h) * d;
            const double *dOt = dO + ((long)t * hq + h) * d;
            double m = -INFINITY;
            for (int a = 0; a < n; ++a) {
              z[a] = scale * dot_dd(qt, k + ((long)u[a] * hkv + g) * d, d);
              if (z[a] > m) m = z[a];
            }
            double den = 0.0;
            for (int a = 0; a < n; ++a) den += exp(z[a] - m);
            for (int e = 0; e < d; ++e) ot[e] = 0.0;
            for (int a = 0; a < n; ++a) {
              P[a] = exp(z[a] - m) / den;
              double gate = exp(lg[slot[a]]);
              const double *vu = v + ((long)u[a] * hkv + g) * d;
              for (int e = 0; e < d; ++e) ot[e] += P[a] * gate * vu[e];
            }
            double D = 0.0;
            for (int e = 0; e < d; ++e) D += dOt[e] * ot[e];
            for (int a = 0; a < n; ++a) {
              const double *ku = k + ((long)u[a] * hkv + g) * d;
              const double *vu = v + ((long)u[a] * hkv + g) * d;
              double gate = exp(lg[slot[a]]);
              double dP = gate * dot_dd(dOt, vu, d);
              double dS = P[a] * (dP - D);
              double *dqt = dq + ((long)t * hq + h) * d;
              double *dku = dk + ((long)u[a] * hkv + g) * d;
              double *dvu = dv + ((long)u[a] * hkv + g) * d;
              for (int e = 0; e < d; ++e) {
                dqt[e] += scale * dS * ku[e];
                dku[e] += scale * dS * qt[e];
                dvu[e] += P[a] * gate * dOt[e];
              }
              dlg[r * Kb + slot[a]] += P[a] * dP;
            }
          }
        }
      }
    }
    free(u);
    free(slot);
    free(z);
    free(P);
    free(ot);
  }
  free(cuqb);
  return 0;
}

/*
 * Gate backward: d logits from d log g through the softmax normaliser
 * ([R] 2-1 g = phi(s); [P] ablation results: the normaliser is shared by all
 * historical blocks).  With p_m = exp(log g_m) over the normaliser set N:
 *   d s_m = [m kept] dlg_m - p_m * sum over kept j of dlg_j     (m in N)
 * GATE_HIST: N = {0..i-1}, the current slot carries no gradient.
 * GATE_ALL:  N = {0..i}, the current block counts as kept.
 * Columns outside N get 0.  Rows are recomputed from the logits.
 */
int sas_oracle_gate_bwd(int nseq, const int32_t *cu, int blk, int hkv, int Kb, int mode,
                        const float *logits, int64_t ld, const int32_t *sel_idx,
                        const double *dlg, double *dlogits) {
  int *cuqb = (int *)malloc(sizeof(int) * (nseq + 1));
  int QB = query_block_offsets(nseq, cu, blk, cuqb);
  long nrows = (long)hkv * QB;
#pragma omp parallel for schedule(dynamic, 8)
  for (long r = 0; r < nrows; ++r) {
    int Q = (int)(r % QB);
    int s = seq_of_qblock(nseq, cuqb, Q);
    int i = Q - cuqb[s];
    const float *sr = logits + r * ld;
    double *out = dlogits + r * ld;
    for (long c = 0; c < ld; ++c) out[c] = 0.0;
    if (mode == ORACLE_GATE_SIGMOID || mode == ORACLE_GATE_RAW) {
      /* independent gates: d s_j = d log g_j * (d log g_j / d s_j), kept
       * history blocks only; d log sigmoid(s) / ds = sigmoid(-s) */
      for (int sl = 0; sl < Kb; ++sl) {
        int j = sel_idx[r * Kb + sl];
        if (j < 0 || j >= i) continue;
        double dl = dlg[r * Kb + sl];
        out[j] += (mode == ORACLE_GATE_RAW) ? dl : dl / (1.0 + exp((double)sr[j]));
      }
      continue;
    }
    int nn = (mode == ORACLE_GATE_ALL) ? i + 1 : i;
    if (nn == 0) continue;
    double m = -INFINITY;
    for (int j = 0; j < nn; ++j)
      if ((double)sr[j] > m) m = (double)sr[j];
    if (m == -INFINITY) continue;
    double acc = 0.0;
    for (int j = 0; j < nn; ++j) acc += exp((double)sr[j] - m);
    double lse = m + log(acc);
    if (mode == ORACLE_GATE_STE) {
      /* straight-through: dL/dg_j (= d log g_j at g = 1) through the soft
       * gate's Jacobian g_j ([j = m] - g_m) */
      double tot_g = 0.0;
      for (int sl = 0; sl < Kb; ++sl) {
        int j = sel_idx[r * Kb + sl];
        if (j < 0 || j >= i) continue;
        double gj = exp((double)sr[j] - lse);
        tot_g += gj * dlg[r * Kb + sl];
        out[j] += gj * dlg[r * Kb + sl];
      }
      for (int j = 0; j < nn; ++j) out[j] -= exp((double)sr[j] - lse) * tot_g;
      continue;
    }
    double tot = 0.0;
    for (int sl = 0; sl < Kb; ++sl) {
      int j = sel_idx[r * Kb + sl];
      if (j < 0) continue;
      if (j == i && mode != ORACLE_GATE_ALL) continue;
      tot += dlg[r * Kb + sl];
      out[j] += dlg[r * Kb + sl];
    }
    for (int j = 0; j < nn; ++j) out[j] -= exp((double)sr[j] - lse) * tot;
  }
  free(cuqb);
  return 0;
}

/* ---------------------------------------------------------------- decode */

/*
 * Reduced-precision summary storage (the pages name bf16 / fp8 summaries as
 * the way to cut the selector scan's bytes): every fp32 value is replaced
 * by the nearest bf16 value, ties to the even one, and returned as the fp32
 * number that bf16 value stands for.  Written from the definition: keep the
 * top 16 bits of the fp32 pattern after adding half a bf16 unit, minus one
 * when the kept part is even (so exact halves go to even).  NaN stays NaN.
 */
int sas_oracle_round_bf16(int64_t n, const float *in, float *out) {
  for (int64_t i = 0; i < n; ++i) {
    uint32_t u;
    memcpy(&u, &in[i], sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) {
      out[i] = in[i];
      continue;
    }
    const uint32_t keep_odd = (u >> 16) & 1u;
    u = (u + 0x7fffu + keep_odd) & 0xffff0000u;
    memcpy(&out[i], &u, sizeof u);
  }
  return 0;
}

/*
 * fp8 summary storage (e4m3: 1 sign bit, 4 exponent bits with bias 7, 3
 * mantissa bits; no infinities, exponent and mantissa all ones = NaN): every
 * fp32 value is replaced by the nearest e4m3 value, ties to the even one,
 * and returned as the fp32 number it stands for.  Written from the
 * definition: below 2^-6 the spacing of the format is 2^-9 (subnormals),
 * in [2^e, 2^(e+1)) with e >= -6 it is 2^(e-3); the value divided by its
 * spacing is rounded to the nearest integer, ties to even (rint in the
 * default rounding mode), and multiplied back (all exact in double).  The
 * largest finite value is 448; a result of 480 or more (the next step of
 * the spacing) has no encoding and becomes NaN, as do infinities and NaN.
 */
int sas_oracle_round_e4m3(int64_t n, const float *in, float *out) {
  for (int64_t i = 0; i < n; ++i) {
    const double x = in[i];
    if (isnan(x) || isinf(x)) {
      out[i] = NAN;
      continue;
    }
    const double a = fabs(x);
    double spacing = ldexp(1.0, -9);
    if (a >= ldexp(1.0, -6)) {
      int e;
      frexp(a, &e); /* a = f 2^e, f in [0.5, 1): a in [2^(e-1), 2^e) */
      spacing = ldexp(1.0, e - 1 - 3);
    }
    const double r = rint(a / spacing) * spacing;
    out[i] = r >= 480.0 ? NAN : (float)copysign(r, x);
  }
  return 0;
}

/*
 * Block summaries of one (sequence, kv head): the mean key of every full
 * history block j < (L-1)/b, in the fixed fp32 order stated in the header
 * ([R] 3-7 step 1: the selector scores cached block summaries).
 * K: [L][d] fp32 values; kbar: [nhist][d].
 */
int sas_oracle_pool_keys_row(int L, int blk, int d, const float *K, float *kbar) {
  int nhist = (L - 1) / blk;
  for (int j = 0; j < nhist; ++j)
    for (int e = 0; e < d; ++e) {
      float acc = 0.0f;
      for (int t = 0; t < blk; ++t) acc = acc + K[(long)(j * blk + t) * d + e];
      kbar[(long)j * d + e] = acc / (float)blk;
    }
  return nhist;
}

/*
 * Coarse summaries for the hierarchical selection (review 7-2: a coarse
 * retrieval narrows the candidate blocks before the selector's final
 * Top-K): super-block J covers history blocks F J .. F J + F - 1, and its
 * summary is the mean of those F block summaries, summed in block order in
 * fp32 and divided by F.  Only complete super-blocks (F J + F - 1 < nhist)
 * have one.  kbar: [nhist][d] (the stored block summaries); cbar:
 * [nhist / F][d].  Returns the number of super-blocks.
 */
int sas_oracle_coarse_summaries(int nhist, int d, int F, const float *kbar, float *cbar) {
  int nsup = nhist / F;
  for (int J = 0; J < nsup; ++J)
    for (int e = 0; e < d; ++e) {
      float acc = 0.0f;
      for (int b = 0; b < F; ++b) acc = acc + kbar[(long)(J * F + b) * d + e];
      cbar[(long)J * d + e] = acc / (float)F;
    }
  return nsup;
}

/*
 * Pooled decode scores of one (sequence, kv head): the group's mean query
 * dotted with each summary, divided by sqrt(d), all in fp32 in the fixed
 * order stated in the header.  q: [G][d]; kbar: [nhist][d]; scores: [nhist].
 */
int sas_oracle_decode_scores_row(int nhist, int d, int G, const float *q, const float *kbar,
                                 float *scores) {
  float *qbar = (float *)malloc(sizeof(float) * d);
  for (int e = 0; e < d; ++e) {
    float acc = 0.0f;
    for (int h = 0; h < G; ++h) acc = acc + q[(long)h * d + e];
    qbar[e] = acc / (float)G;
  }
  float rs = sqrtf((float)d);
  for (int j = 0; j < nhist; ++j) {
    float acc = 0.0f;
    for (int e = 0; e < d; ++e) acc = fmaf(qbar[e], kbar[(long)j * d + e], acc);
    scores[j] = acc / rs;
  }
  free(qbar);
  return 0;
}

/*
 * Decode attention of one (sequence, kv head) for its G query heads
 * ([R] 3-7 steps 3-4): the kept history blocks (whole) plus the present
 * tokens of the current block, log gates added per block.
 * q: [G][d]; K, V: [L][d]; sel_idx / sel_lg: [Kb] (sel_lg NULL: no gate);
 * o: [G][d]; lse: [G].
 */
int sas_oracle_decode_row(int L, int blk, int d, int G, int Kb, double scale, const double *q,
                          const double *K, const double *V, const int32_t *sel_idx,
                          const double *sel_lg, double *o, double *lse) {
  int cur = (L - 1) / blk;
  int maxkeys = Kb * blk;
  int *u = (int *)malloc(sizeof(int) * maxkeys);
  int *slot = (int *)malloc(sizeof(int) * maxkeys);
  double *z = (double *)malloc(sizeof(double) * maxkeys);
  int n = attended_keys(sel_idx, Kb, cur, blk, 0, L, L - 1, u, slot);
  for (int h = 0; h < G; ++h) {
    double m = -INFINITY;
    for (int a = 0; a < n; ++a) {
      z[a] = scale * dot_dd(q + (long)h * d, K + (long)u[a] * d, d) +
             (sel_lg ? sel_lg[slot[a]] : 0.0);
      if (z[a] > m) m = z[a];
    }
    double den = 0.0;
    for (int a = 0; a < n; ++a) den += exp(z[a] - m);
    for (int e = 0; e < d; ++e) o[(long)h * d + e] = 0.0;
    for (int a = 0; a < n; ++a) {
      double p = exp(z[a] - m) / den;
      for (int e = 0; e < d; ++e) o[(long)h * d + e] += p * V[(long)u[a] * d + e];
    }
    lse[h] = m + log(den);
  }
  free(u);
  free(slot);
  free(z);
  return n;
}
