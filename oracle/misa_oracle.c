/*
 * misa_oracle.c -- plain CPU oracle for the DSA indexer, MISA and MISA-dagger.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg load this library.  The GPU path never
 * calls it, links it or includes anything from it, and it shares no code,
 * header, table or helper with the GPU path.
 *
 * Every bf16 or fp32 input is widened exactly to double and every sum is
 * accumulated in double, in a fixed order (dimension c ascending, then head j
 * ascending, then block b ascending).  The code follows the definitions
 * step by step; there is no blocking, fusion or reordering.
 *
 * Sources, cited by page title and section:
 *   [MISA-TS]  "MISA: Mixture of Indexer Sparse Attention for Long-Context
 *              LLM Inference" (gist.science explainer), Technical Summary:
 *              "Problem Statement", "Methodology: MISA",
 *              "Hierarchical Variant (MISA†)".
 *   [MISA-AB]  The MISA abstract, printed on the thelatestinai page titled
 *              "HISA: Efficient Hierarchical Indexing for Fine-Grained
 *              Sparse Attention" (first paragraph).
 *   [HISA-AB]  "HISA" abstract on the Lattice page for arXiv 2603.28458, and
 *              the aiqbench page "HISA: Efficient Hierarchical Indexing for
 *              Fine-Grained Sparse Attention" (v4 abstract).
 *
 * Readings taken where the pages are silent (each is repeated at its use):
 *   R1  the prefix of a query at position p is tokens 0..p (inclusive);
 *   R3  the indexer score is I(i) = sum_j w_j * max(0, q_j . k_i), no scale;
 *   R4  blocks start at token 0; a partial last block is the mean over the
 *       prefix tokens it holds;
 *   R5  router affinity = ReLU(q_j . Kbar_b), aggregated by a sum over the
 *       query's blocks and multiplied by w_j (mode 0) or |w_j| (mode 1);
 *   R6  ties: larger value first, then the lower index; -0.0 equals +0.0.
 *   H1-H4  the hierarchical indexer's readings, at orc_hisa.
 * The pages do not fix the functional forms R3 and R5: these readings are
 * this implementation's, and the tests pin the code to them (closed forms,
 * brute force, invariants, a hand-worked example), not to the pages.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_EINVAL -1
#define ORC_ENOMEM -2

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
static double orc_bf16(uint16_t u) {
  uint32_t x = ((uint32_t)u) << 16;
  float f;
  memcpy(&f, &x, sizeof f);
  return (double)f;
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ------------------------------------------------------------------------- */
/* Ranking: sort by (value descending, index ascending).  [MISA-TS] Problem  */
/* Statement: the indexer keeps the top-k tokens; tie rule is reading R6.    */
/* ------------------------------------------------------------------------- */
typedef struct {
  double v;
  int64_t i;
} orc_item;

static int orc_cmp(const void *pa, const void *pb) {
  const orc_item *a = (const orc_item *)pa, *b = (const orc_item *)pb;
  if (a->v > b->v) return -1;  /* -0.0 and +0.0 compare equal here */
  if (a->v < b->v) return 1;
  return (a->i < b->i) ? -1 : (a->i > b->i) ? 1 : 0;
}

/*
 * orc_topk: the first min(k, n) indices i in [0, n) ordered by
 * (v[i] desc, i asc); slots beyond n are padded with -1.  idx_out has k
 * entries; when val_out is non-NULL it receives v[idx] (or -inf for pads).
 */
int orc_topk(const double *v, int64_t n, int64_t k, int32_t *idx_out,
             double *val_out) {
  if (n < 0 || k < 0 || (n > 0 && !v) || (k > 0 && !idx_out)) return ORC_EINVAL;
  orc_item *it = (orc_item *)malloc(sizeof(orc_item) * (size_t)(n > 0 ? n : 1));
  if (!it) return ORC_ENOMEM;
  for (int64_t i = 0; i < n; ++i) {
    it[i].v = v[i];
    it[i].i = i;
  }
  qsort(it, (size_t)n, sizeof(orc_item), orc_cmp);
  for (int64_t r = 0; r < k; ++r) {
    if (r < n) {
      idx_out[r] = (int32_t)it[r].i;
      if (val_out) val_out[r] = it[r].v;
    } else {
      idx_out[r] = -1;
      if (val_out) val_out[r] = -INFINITY;
    }
  }
  free(it);
  return ORC_OK;
}

/* Same ranking over fp32 values (the GPU's own precision): widening to
 * double is exact and preserves the order, so this is orc_topk on them. */
int orc_topk_f32(const float *v, int64_t n, int64_t k, int32_t *idx_out) {
  if (n < 0 || (n > 0 && !v)) return ORC_EINVAL;
  double *dv = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  if (!dv) return ORC_ENOMEM;
  for (int64_t i = 0; i < n; ++i) dv[i] = (double)v[i];
  int rc = orc_topk(dv, n, k, idx_out, NULL);
  free(dv);
  return rc;
}

/* ------------------------------------------------------------------------- */
/* Head-token dot product x_j(i) = sum_c q_j[c] * k_i[c].                    */
/* [MISA-TS] Key Contributions: the per-token head-token products.           */
/* ------------------------------------------------------------------------- */
static double orc_dot_bf16(const uint16_t *qv, const uint16_t *kv, int d) {
  double s = 0.0;
  for (int c = 0; c < d; ++c) s += orc_bf16(qv[c]) * orc_bf16(kv[c]);
  return s;
}

static int orc_cmp_int(const void *pa, const void *pb) {
  int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
  return (a < b) ? -1 : (a > b) ? 1 : 0;
}

/*
 * orc_scores: indexer scores of every prefix key, for every query row t.
 *   keys   bf16 [S][Lmax][d]      q  bf16 [T][H][d]      w  fp32 [T][H]
 *   q_seq  [T] sequence of row t  q_pos [T] position p_t (prefix = 0..p_t, R1)
 *   heads  NULL -> all H heads (the DSA indexer, [MISA-TS] Problem Statement)
 *          else [T][h] head ids (the routed heads, [MISA-TS] Methodology:
 *          Sparse Token Scoring); the sum runs over the set in ascending id.
 *   out    double [T][Lmax]: I(i) = sum_j w_j * max(0, x_j(i)) for i <= p_t
 *          (reading R3), -inf for i > p_t.
 */
int orc_scores(const uint16_t *keys, const uint16_t *q, const float *w,
               const int32_t *q_seq, const int32_t *q_pos, int S, int Lmax,
               int d, int T, int H, const int32_t *heads, int h, double *out) {
  if (!keys || !q || !w || !q_seq || !q_pos || !out) return ORC_EINVAL;
  if (S < 1 || Lmax < 1 || d < 1 || T < 0 || H < 1) return ORC_EINVAL;
  if (heads && (h < 1 || h > H)) return ORC_EINVAL;
  int nh = heads ? h : H;
  int32_t *hs = (int32_t *)malloc(sizeof(int32_t) * (size_t)T * (size_t)nh + 1);
  if (!hs) return ORC_ENOMEM;
  for (int t = 0; t < T; ++t) {
    if (q_seq[t] < 0 || q_seq[t] >= S || q_pos[t] < 0 || q_pos[t] >= Lmax) {
      free(hs);
      return ORC_EINVAL;
    }
    for (int r = 0; r < nh; ++r) {
      int32_t j = heads ? heads[(size_t)t * h + r] : r;
      if (j < 0 || j >= H) {
        free(hs);
        return ORC_EINVAL;
      }
      hs[(size_t)t * nh + r] = j;
    }
    qsort(hs + (size_t)t * nh, (size_t)nh, sizeof(int32_t), orc_cmp_int);
  }
  int64_t total = (int64_t)T * Lmax;
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < total; ++e) {
    int t = (int)(e / Lmax);
    int i = (int)(e % Lmax);
    if (i > q_pos[t]) {
      out[e] = -INFINITY;
      continue;
    }
    const uint16_t *kv = keys + ((size_t)q_seq[t] * Lmax + i) * d;
    double s = 0.0;
    for (int r = 0; r < nh; ++r) {
      int j = hs[(size_t)t * nh + r];
      double x = orc_dot_bf16(q + ((size_t)t * H + j) * d, kv, d);
      s += (double)w[(size_t)t * H + j] * (x > 0.0 ? x : 0.0);
    }
    out[e] = s;
  }
  free(hs);
  return ORC_OK;
}

/*
 * orc_pool: mean-pooled indexing keys of each sequence.
 * [MISA-TS] Methodology: Lightweight Block-Pooled Router -- the prefix is cut
 * into M = ceil(L/B) blocks summarised by mean-pooled indexing keys.
 * Reading R4: block b holds tokens [bB, min(bB+B, len)); its mean is over
 * the tokens present.  A block with no token present is written as zeros.
 *   pooled double [S][ceil(Lmax/B)][d]
 */
int orc_pool(const uint16_t *keys, const int32_t *seq_lens, int S, int Lmax,
             int d, int B, double *pooled) {
  if (!keys || !seq_lens || !pooled || S < 1 || Lmax < 1 || d < 1 || B < 1)
    return ORC_EINVAL;
  int Mmax = (Lmax + B - 1) / B;
  for (int s = 0; s < S; ++s)
    if (seq_lens[s] < 0 || seq_lens[s] > Lmax) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t sb = 0; sb < (int64_t)S * Mmax; ++sb) {
    int s = (int)(sb / Mmax);
    int b = (int)(sb % Mmax);
    int lo = b * B;
    int hi = lo + B < seq_lens[s] ? lo + B : seq_lens[s];
    double *dst = pooled + (size_t)sb * d;
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int i = lo; i < hi; ++i)
        acc += orc_bf16(keys[((size_t)s * Lmax + i) * d + c]);
      dst[c] = hi > lo ? acc / (double)(hi - lo) : 0.0;
    }
  }
  return ORC_OK;
}

/*
 * orc_route: the block-pooled head router of one query row.
 * [MISA-TS] Methodology: Lightweight Block-Pooled Router -- per-head
 * affinities against the mean-pooled keys of the query's M = ceil(n/B)
 * prefix blocks, aggregated into one importance per head; the top-h heads
 * are kept.  [MISA-AB]: a query-dependent subset of heads.
 * Readings R1, R4, R5, R6.  The last block of the prefix is the mean of the
 * prefix tokens in it (the query's own partial block).
 *   g      double [T][H]  g_j = w'_j * sum_b max(0, q_j . Kbar_b),
 *                         w' = w (mode 0) or |w| (mode 1)
 *   heads  [T][h]         the first h heads by (g desc, j asc), in that order
 */
int orc_route(const uint16_t *keys, const uint16_t *q, const float *w,
              const int32_t *q_seq, const int32_t *q_pos, int S, int Lmax,
              int d, int T, int H, int B, int h, int mode, double *g,
              int32_t *heads) {
  if (!keys || !q || !w || !q_seq || !q_pos || !g || !heads) return ORC_EINVAL;
  if (S < 1 || Lmax < 1 || d < 1 || T < 0 || H < 1 || B < 1 || h < 1 ||
      h > H || (mode != 0 && mode != 1))
    return ORC_EINVAL;
  for (int t = 0; t < T; ++t)
    if (q_seq[t] < 0 || q_seq[t] >= S || q_pos[t] < 0 || q_pos[t] >= Lmax)
      return ORC_EINVAL;
  int rc = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int t = 0; t < T; ++t) {
    int n = q_pos[t] + 1;
    int M = (n + B - 1) / B;
    const uint16_t *ks = keys + (size_t)q_seq[t] * Lmax * d;
    double *kbar = (double *)malloc(sizeof(double) * (size_t)M * d);
    double *agg = (double *)calloc((size_t)H, sizeof(double));
    int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)h);
    if (!kbar || !agg || !sel) {
#pragma omp atomic write
      rc = ORC_ENOMEM;
      free(kbar); free(agg); free(sel);
      continue;
    }
    for (int b = 0; b < M; ++b) {
      int lo = b * B, hi = lo + B < n ? lo + B : n;
      for (int c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int i = lo; i < hi; ++i) acc += orc_bf16(ks[(size_t)i * d + c]);
        kbar[(size_t)b * d + c] = acc / (double)(hi - lo);
      }
    }
    for (int j = 0; j < H; ++j) {
      const uint16_t *qj = q + ((size_t)t * H + j) * d;
      double sum = 0.0;
      for (int b = 0; b < M; ++b) {
        double a = 0.0;
        for (int c = 0; c < d; ++c) a += orc_bf16(qj[c]) * kbar[(size_t)b * d + c];
        sum += a > 0.0 ? a : 0.0;
      }
      double wj = (double)w[(size_t)t * H + j];
      if (mode == 1) wj = fabs(wj);
      agg[j] = wj * sum;
      g[(size_t)t * H + j] = agg[j];
    }
    if (orc_topk(agg, H, h, sel, NULL) != ORC_OK) {
#pragma omp atomic write
      rc = ORC_ENOMEM;
    } else {
      memcpy(heads + (size_t)t * h, sel, sizeof(int32_t) * (size_t)h);
    }
    free(kbar); free(agg); free(sel);
  }
  return rc;
}

/* Per-row selection over a score matrix: top-k of row t's prefix. */
static int orc_select_rows(const double *scores, const int32_t *q_pos, int T,
                           int Lmax, int k, int32_t *idx, double *val) {
  int rc = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int t = 0; t < T; ++t) {
    int r = orc_topk(scores + (size_t)t * Lmax, (int64_t)q_pos[t] + 1, k,
                     idx + (size_t)t * k, val ? val + (size_t)t * k : NULL);
    if (r != ORC_OK) {
#pragma omp atomic write
      rc = r;
    }
  }
  return rc;
}

/*
 * orc_dsa: the dense DSA indexer -- every prefix key scored by all H heads,
 * then the per-query top-k ([MISA-TS] Problem Statement; [MISA-AB]: all
 * heads share one selected token set).
 *   idx [T][k], val [T][k] (may be NULL), scores [T][Lmax] (may be NULL)
 */
int orc_dsa(const uint16_t *keys, const uint16_t *q, const float *w,
            const int32_t *q_seq, const int32_t *q_pos, int S, int Lmax, int d,
            int T, int H, int k, int32_t *idx, double *val, double *scores) {
  if (!idx || k < 1) return ORC_EINVAL;
  double *sc = scores ? scores : (double *)malloc(sizeof(double) * (size_t)T * Lmax + 1);
  if (!sc) return ORC_ENOMEM;
  int rc = orc_scores(keys, q, w, q_seq, q_pos, S, Lmax, d, T, H, NULL, 0, sc);
  if (rc == ORC_OK) rc = orc_select_rows(sc, q_pos, T, Lmax, k, idx, val);
  if (!scores) free(sc);
  return rc;
}

/*
 * orc_misa: router -> routed-head token scoring -> top-k
 * ([MISA-TS] Methodology: MISA, both stages).
 *   heads [T][h] and g [T][H] receive the router's outputs (g may be NULL).
 */
int orc_misa(const uint16_t *keys, const uint16_t *q, const float *w,
             const int32_t *q_seq, const int32_t *q_pos, int S, int Lmax,
             int d, int T, int H, int B, int h, int mode, int k, int32_t *heads,
             double *g, int32_t *idx, double *val, double *scores) {
  if (!idx || !heads || k < 1) return ORC_EINVAL;
  double *gg = g ? g : (double *)malloc(sizeof(double) * (size_t)T * H + 1);
  double *sc = scores ? scores : (double *)malloc(sizeof(double) * (size_t)T * Lmax + 1);
  int rc = (gg && sc) ? ORC_OK : ORC_ENOMEM;
  if (rc == ORC_OK)
    rc = orc_route(keys, q, w, q_seq, q_pos, S, Lmax, d, T, H, B, h, mode, gg, heads);
  if (rc == ORC_OK)
    rc = orc_scores(keys, q, w, q_seq, q_pos, S, Lmax, d, T, H, heads, h, sc);
  if (rc == ORC_OK) rc = orc_select_rows(sc, q_pos, T, Lmax, k, idx, val);
  if (!g) free(gg);
  if (!scores) free(sc);
  return rc;
}

/*
 * orc_rerank: the fine stage of MISA-dagger.  [MISA-TS] Hierarchical Variant
 * (MISA†), Fine Stage: the original all-head DSA indexer rescores only the
 * candidate tokens, and the top-k of them is kept.  cand [T][kc] holds token
 * ids, -1 for an empty slot.  The scores are recomputed with all H heads
 * (reading R3); ranking is (score desc, token id asc), padded with -1.
 */
int orc_rerank(const uint16_t *keys, const uint16_t *q, const float *w,
               const int32_t *q_seq, const int32_t *q_pos, int S, int Lmax,
               int d, int T, int H, const int32_t *cand, int kc, int k,
               int32_t *idx, double *val) {
  if (!keys || !q || !w || !q_seq || !q_pos || !cand || !idx || kc < 1 || k < 1)
    return ORC_EINVAL;
  int rc = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int t = 0; t < T; ++t) {
    const int32_t *ct = cand + (size_t)t * kc;
    int nv = 0;
    orc_item *it = (orc_item *)malloc(sizeof(orc_item) * (size_t)kc);
    if (!it) {
#pragma omp atomic write
      rc = ORC_ENOMEM;
      continue;
    }
    for (int r = 0; r < kc; ++r) {
      int32_t i = ct[r];
      if (i < 0) continue;
      if (i > q_pos[t]) { /* a candidate outside the prefix is invalid input */
#pragma omp atomic write
        rc = ORC_EINVAL;
        continue;
      }
      const uint16_t *kv = keys + ((size_t)q_seq[t] * Lmax + i) * d;
      double s = 0.0;
      for (int j = 0; j < H; ++j) {
        double x = orc_dot_bf16(q + ((size_t)t * H + j) * d, kv, d);
        s += (double)w[(size_t)t * H + j] * (x > 0.0 ? x : 0.0);
      }
      it[nv].v = s;
      it[nv].i = i;
      ++nv;
    }
    qsort(it, (size_t)nv, sizeof(orc_item), orc_cmp);
    for (int r = 0; r < k; ++r) {
      idx[(size_t)t * k + r] = r < nv ? (int32_t)it[r].i : -1;
      if (val) val[(size_t)t * k + r] = r < nv ? it[r].v : -INFINITY;
    }
    free(it);
  }
  return rc;
}

/*
 * orc_misa_dagger: MISA-dagger, coarse to fine.  [MISA-TS] Hierarchical
 * Variant (MISA†): the routed pass keeps k' candidates (Coarse Stage), then
 * the all-head indexer rescores them and keeps the top-k (Fine Stage).
 *   cand [T][kc] receives the coarse candidate set (may be NULL).
 */
int orc_misa_dagger(const uint16_t *keys, const uint16_t *q, const float *w,
                    const int32_t *q_seq, const int32_t *q_pos, int S, int Lmax,
                    int d, int T, int H, int B, int h, int mode, int kc, int k,
                    int32_t *heads, int32_t *cand, int32_t *idx, double *val) {
  if (!idx || !heads || kc < 1 || k < 1) return ORC_EINVAL;
  int32_t *cc = cand ? cand : (int32_t *)malloc(sizeof(int32_t) * (size_t)T * kc + 1);
  if (!cc) return ORC_ENOMEM;
  int rc = orc_misa(keys, q, w, q_seq, q_pos, S, Lmax, d, T, H, B, h, mode, kc,
                    heads, NULL, cc, NULL, NULL);
  if (rc == ORC_OK)
    rc = orc_rerank(keys, q, w, q_seq, q_pos, S, Lmax, d, T, H, cc, kc, k, idx, val);
  if (!cand) free(cc);
  return rc;
}

/*
 * orc_hisa: the hierarchical block-to-token indexer ([HISA-AB], the
 * abstract: a first pass ranks whole blocks by a score on each block's pooled
 * summary and drops the low-ranked ones; the unchanged token-level indexer
 * then scores only the tokens of the surviving blocks, and its per-query
 * top-k token set stays the output).  Readings, the pages giving no formula:
 *   H1  a block's representation is the mean of its keys (R4's blocks, as
 *       MISA's router pools them); the query's own last block is the mean
 *       over its prefix tokens;
 *   H2  a block's score is the indexer's score form on that mean:
 *       s_b = sum_{j in heads} w_j * max(0, q_j . Kbar_b), j ascending;
 *   H3  the m blocks with the largest s_b are kept (R6 ties: lower block id);
 *       m is a parameter, the pages giving no number;
 *   H4  every prefix token of the kept blocks is scored with the same heads
 *       (R3) and the top-k by R6 is the output, padded with -1.
 * heads == NULL: all H heads (HISA).  heads [T][h]: those heads in both
 * stages (the routed heads of MISA, for MISA composed with HISA).
 *   idx [T][k]; val [T][k], blocks [T][m] (-1 padded) and
 *   bscore [T][ceil(Lmax/B)] (-inf past the query's blocks) may be NULL.
 */
int orc_hisa(const uint16_t *keys, const uint16_t *q, const float *w,
             const int32_t *q_seq, const int32_t *q_pos, int S, int Lmax, int d,
             int T, int H, int B, int m, const int32_t *heads, int h, int k,
             int32_t *idx, double *val, int32_t *blocks, double *bscore) {
  if (!keys || !q || !w || !q_seq || !q_pos || !idx) return ORC_EINVAL;
  if (S < 1 || Lmax < 1 || d < 1 || T < 0 || H < 1 || B < 1 || m < 1 || k < 1)
    return ORC_EINVAL;
  if (heads && (h < 1 || h > H)) return ORC_EINVAL;
  const int nh = heads ? h : H;
  const int Mmax = (Lmax + B - 1) / B;
  for (int t = 0; t < T; ++t) {
    if (q_seq[t] < 0 || q_seq[t] >= S || q_pos[t] < 0 || q_pos[t] >= Lmax) return ORC_EINVAL;
    for (int r = 0; heads && r < h; ++r)
      if (heads[(size_t)t * h + r] < 0 || heads[(size_t)t * h + r] >= H) return ORC_EINVAL;
  }
  int rc = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int t = 0; t < T; ++t) {
    const int n = q_pos[t] + 1;
    const int M = (n + B - 1) / B;
    const uint16_t *ks = keys + (size_t)q_seq[t] * Lmax * d;
    int32_t *hs = (int32_t *)malloc(sizeof(int32_t) * (size_t)nh);
    double *kbar = (double *)malloc(sizeof(double) * (size_t)M * d);
    double *s = (double *)malloc(sizeof(double) * (size_t)M);
    int32_t *kept = (int32_t *)malloc(sizeof(int32_t) * (size_t)m);
    orc_item *it = (orc_item *)malloc(sizeof(orc_item) * ((size_t)m * B + 1));
    if (!hs || !kbar || !s || !kept || !it) {
#pragma omp atomic write
      rc = ORC_ENOMEM;
      free(hs); free(kbar); free(s); free(kept); free(it);
      continue;
    }
    for (int r = 0; r < nh; ++r) hs[r] = heads ? heads[(size_t)t * h + r] : r;
    qsort(hs, (size_t)nh, sizeof(int32_t), orc_cmp_int);
    /* H1: block means; the last block holds the prefix tokens in it */
    for (int b = 0; b < M; ++b) {
      int lo = b * B, hi = lo + B < n ? lo + B : n;
      for (int c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int i = lo; i < hi; ++i) acc += orc_bf16(ks[(size_t)i * d + c]);
        kbar[(size_t)b * d + c] = acc / (double)(hi - lo);
      }
    }
    /* H2: block scores */
    for (int b = 0; b < M; ++b) {
      double sb = 0.0;
      for (int r = 0; r < nh; ++r) {
        const int j = hs[r];
        const uint16_t *qj = q + ((size_t)t * H + j) * d;
        double x = 0.0;
        for (int c = 0; c < d; ++c) x += orc_bf16(qj[c]) * kbar[(size_t)b * d + c];
        sb += (double)w[(size_t)t * H + j] * (x > 0.0 ? x : 0.0);
      }
      s[b] = sb;
    }
    if (bscore)
      for (int b = 0; b < Mmax; ++b) bscore[(size_t)t * Mmax + b] = b < M ? s[b] : -INFINITY;
    /* H3: the m best blocks */
    if (orc_topk(s, M, m, kept, NULL) != ORC_OK) {
#pragma omp atomic write
      rc = ORC_ENOMEM;
    } else {
      if (blocks) memcpy(blocks + (size_t)t * m, kept, sizeof(int32_t) * (size_t)m);
      /* H4: the indexer over the kept blocks' prefix tokens */
      int nv = 0;
      for (int r = 0; r < m; ++r) {
        const int b = kept[r];
        if (b < 0) continue;
        const int lo = b * B, hi = lo + B < n ? lo + B : n;
        for (int i = lo; i < hi; ++i) {
          const uint16_t *kv = ks + (size_t)i * d;
          double si = 0.0;
          for (int rr = 0; rr < nh; ++rr) {
            const int j = hs[rr];
            double x = orc_dot_bf16(q + ((size_t)t * H + j) * d, kv, d);
            si += (double)w[(size_t)t * H + j] * (x > 0.0 ? x : 0.0);
          }
          it[nv].v = si;
          it[nv].i = i;
          ++nv;
        }
      }
      qsort(it, (size_t)nv, sizeof(orc_item), orc_cmp);
      for (int r = 0; r < k; ++r) {
        idx[(size_t)t * k + r] = r < nv ? (int32_t)it[r].i : -1;
        if (val) val[(size_t)t * k + r] = r < nv ? it[r].v : -INFINITY;
      }
    }
    free(hs); free(kbar); free(s); free(kept); free(it);
  }
  return rc;
}
