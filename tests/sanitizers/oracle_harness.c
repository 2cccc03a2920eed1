/*
 * Runs every oracle entry point on small ragged problems, built with
 * AddressSanitizer and UndefinedBehaviorSanitizer, buffers allocated at
 * exactly their documented sizes, so any out-of-bounds access or undefined
 * operation in the oracle is reported.  Also checks two exact invariants on
 * the way (each log-gate-gradient row sums to zero; the gate backward of a
 * row sums to zero).  Exit status 0 = clean.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int sas_oracle_num_qblocks(int nseq, const int32_t *cu, int blk);
int sas_oracle_gate_topk(int nseq, const int32_t *cu, int blk, int hkv, int Kb, int mode,
                         const float *logits, int64_t ld, int32_t *sel_idx, double *sel_lg,
                         double *gate_lse);
int sas_oracle_gate_row(const float *scores, int i, int Kb, int mode, int32_t *idx, double *lg,
                        double *lse);
int sas_oracle_fwd(int nseq, const int32_t *cu, int blk, int hq, int hkv, int d, int Kb,
                   double scale, const double *q, const double *k, const double *v,
                   const int32_t *sel_idx, const double *sel_lg, const unsigned char *row_mask,
                   double *o, double *lse);
int sas_oracle_bwd(int nseq, const int32_t *cu, int blk, int hq, int hkv, int d, int Kb,
                   double scale, const double *q, const double *k, const double *v,
                   const double *dO, const int32_t *sel_idx, const double *sel_lg,
                   const unsigned char *row_mask, const unsigned char *kblk_mask, double *dq,
                   double *dk, double *dv, double *dlg);
int sas_oracle_fwd_outer(int nseq, const int32_t *cu, int blk, int hq, int hkv, int d, int Kb,
                         double scale, const double *q, const double *k, const double *v,
                         const int32_t *sel_idx, const double *sel_lg, double *o, double *lse);
int sas_oracle_bwd_outer(int nseq, const int32_t *cu, int blk, int hq, int hkv, int d, int Kb,
                         double scale, const double *q, const double *k, const double *v,
                         const double *dO, const int32_t *sel_idx, const double *sel_lg,
                         double *dq, double *dk, double *dv, double *dlg);
int sas_oracle_gate_bwd(int nseq, const int32_t *cu, int blk, int hkv, int Kb, int mode,
                        const float *logits, int64_t ld, const int32_t *sel_idx,
                        const double *dlg, double *dlogits);
int sas_oracle_round_bf16(int64_t n, const float *in, float *out);
int sas_oracle_pool_keys_row(int L, int blk, int d, const float *K, float *kbar);
int sas_oracle_decode_scores_row(int nhist, int d, int G, const float *q, const float *kbar,
                                 float *scores);
int sas_oracle_decode_row(int L, int blk, int d, int G, int Kb, double scale, const double *q,
                          const double *K, const double *V, const int32_t *sel_idx,
                          const double *sel_lg, double *o, double *lse);

static uint64_t state = 88172645463325252ull;
static double rnd(void) { /* xorshift64, uniform in [-1, 1) */
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return (double)(state >> 11) / (double)(1ull << 52) - 1.0;
}
static double *dvec(size_t n) {
  double *x = malloc(sizeof(double) * (n ? n : 1));
  for (size_t i = 0; i < n; ++i) x[i] = rnd();
  return x;
}
static float *fvec(size_t n, double s) {
  float *x = malloc(sizeof(float) * (n ? n : 1));
  for (size_t i = 0; i < n; ++i) x[i] = (float)(s * rnd());
  return x;
}

static int failures = 0;

int main(void) {
  enum { NSEQ = 3, BLK = 4, HQ = 4, HKV = 2, D = 8, KB = 3 };
  const int32_t cu[NSEQ + 1] = {0, 23, 31, 32}; /* 6, 2 and 1 blocks, ragged */
  const int T = cu[NSEQ];
  const int QB = sas_oracle_num_qblocks(NSEQ, cu, BLK);
  const int ld = 6;
  double *q = dvec((size_t)T * HQ * D), *k = dvec((size_t)T * HKV * D);
  double *v = dvec((size_t)T * HKV * D), *dO = dvec((size_t)T * HQ * D);
  float *logits = fvec((size_t)HKV * QB * ld, 2.0);
  logits[3] = -INFINITY;
  for (int mode = 0; mode <= 4; ++mode) {
    int32_t *idx = malloc(sizeof(int32_t) * HKV * QB * KB);
    double *lg = malloc(sizeof(double) * HKV * QB * KB), *glse = malloc(sizeof(double) * HKV * QB);
    if (sas_oracle_gate_topk(NSEQ, cu, BLK, HKV, KB, mode, logits, ld, idx, lg, glse)) ++failures;
    double *o = malloc(sizeof(double) * T * HQ * D), *lse = malloc(sizeof(double) * T * HQ);
    unsigned char *rm = calloc((size_t)HKV * QB, 1);
    rm[1] = rm[QB + 2] = 1;
    if (sas_oracle_fwd(NSEQ, cu, BLK, HQ, HKV, D, KB, 0.35, q, k, v, idx, lg, NULL, o, lse))
      ++failures;
    if (sas_oracle_fwd(NSEQ, cu, BLK, HQ, HKV, D, KB, 0.35, q, k, v, idx, lg, rm, o, lse))
      ++failures;
    double *dq = malloc(sizeof(double) * T * HQ * D), *dk = malloc(sizeof(double) * T * HKV * D);
    double *dv = malloc(sizeof(double) * T * HKV * D), *dlg = malloc(sizeof(double) * HKV * QB * KB);
    if (sas_oracle_bwd(NSEQ, cu, BLK, HQ, HKV, D, KB, 0.35, q, k, v, dO, idx, lg, rm, rm, dq, dk,
                       dv, dlg))
      ++failures;
    if (sas_oracle_bwd(NSEQ, cu, BLK, HQ, HKV, D, KB, 0.35, q, k, v, dO, idx, lg, NULL, NULL, dq,
                       dk, dv, dlg))
      ++failures;
    for (int r = 0; r < HKV * QB; ++r) {
      double s = 0.0;
      for (int c = 0; c < KB; ++c) s += dlg[r * KB + c];
      if (mode == 0 && fabs(s) > 1e-9) {
        printf("FAIL dlg row %d sums to %g\n", r, s);
        ++failures;
      }
    }
    double *dz = malloc(sizeof(double) * HKV * QB * ld);
    sas_oracle_gate_bwd(NSEQ, cu, BLK, HKV, KB, mode, logits, ld, idx, dlg, dz);
    sas_oracle_fwd_outer(NSEQ, cu, BLK, HQ, HKV, D, KB, 0.35, q, k, v, idx, lg, o, lse);
    sas_oracle_bwd_outer(NSEQ, cu, BLK, HQ, HKV, D, KB, 0.35, q, k, v, dO, idx, lg, dq, dk, dv,
                         dlg);
    free(idx); free(lg); free(glse); free(o); free(lse); free(rm);
    free(dq); free(dk); free(dv); free(dlg); free(dz);
  }
  /* decode path: one row of L tokens, G heads */
  for (int L = 1; L <= 23; L += 11) {
    const int G = HQ / HKV, nhist = (L - 1) / BLK;
    float *Kf = fvec((size_t)L * D, 1.0), *qf = fvec((size_t)G * D, 1.0);
    float *kbar = malloc(sizeof(float) * (nhist ? nhist : 1) * D), *rb = malloc(sizeof(float) * L * D);
    sas_oracle_round_bf16((int64_t)L * D, Kf, rb);
    sas_oracle_pool_keys_row(L, BLK, D, Kf, kbar);
    float *sc = malloc(sizeof(float) * (nhist + 1));
    sas_oracle_decode_scores_row(nhist, D, G, qf, kbar, sc);
    sc[nhist] = 0.f;
    int32_t idx[KB];
    double lg[KB], lse;
    sas_oracle_gate_row(sc, nhist, KB, 0, idx, lg, &lse);
    double *Kd = dvec((size_t)L * D), *Vd = dvec((size_t)L * D), *qd = dvec((size_t)G * D);
    double o[HQ * D], olse[HQ];
    sas_oracle_decode_row(L, BLK, D, G, KB, 0.35, qd, Kd, Vd, idx, lg, o, olse);
    sas_oracle_decode_row(L, BLK, D, G, KB, 0.35, qd, Kd, Vd, idx, NULL, o, olse);
    free(Kf); free(qf); free(kbar); free(rb); free(sc); free(Kd); free(Vd); free(qd);
  }
  free(q); free(k); free(v); free(dO); free(logits);
  printf("oracle harness: %d failures\n", failures);
  return failures ? 1 : 0;
}
