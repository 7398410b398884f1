/*
 * MoBA forward pass -- plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code with
 * the GPU path and must never be used to produce a product result.
 *
 * Sources (cited by page title and section):
 *  [S] "MoBA: Mixture of Block Attention for Long-Context LLMs", summary page on
 *      paper-graph-ui.vercel.app, section 3.4 "Detailed, Sentence-Based
 *      Technical Breakdown" and its sub-headings.
 *  [R] the paperhub.cn review page for the same paper, authors' rebuttal (W1).
 *  [C] "MoBA (Mixture of Block Attention)" concept note (research-hub),
 *      "Key math / How it works".
 *
 * Layout (packed variable-length batch, "THD"):
 *   q[T][Hq][d], k[T][Hkv][d], v[T][Hkv][d]; elements are fp32, or bf16 given
 *   as raw 16-bit patterns; both are widened to double exactly.
 *   cu_seqlens[S+1]: sequence s owns rows [cu[s], cu[s+1]).
 *
 * Readings taken where the pages are silent or disagree (listed in the design
 * notes as well):
 *   - blocks are 0-indexed per sequence: block j of a sequence of length L
 *     covers local rows [jB, min((j+1)B, L)); the last block may be short;
 *   - the query's own block c is always selected and counts toward k, so at
 *     most k-1 earlier blocks are picked by score;
 *   - candidates for the score-based pick are blocks j < c only (future blocks
 *     are -inf and the current block is forced);
 *   - ties in score are broken by the lower block index;
 *   - the gate score is the raw inner product (no temperature); attention
 *     logits use the caller's softmax scale (1/sqrt(d) by default);
 *   - each query head selects its own blocks; query head h reads kv head
 *     h / (Hq/Hkv);
 *   - lse is the natural-log log-sum-exp of the scaled logits.
 *
 * Pinned by tests/test_oracle_pins.py (dense special case, block-local case,
 * brute-force subset search, explicit-mask softmax, closed forms, varlen and
 * merge identities, printed sparsities).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double load_elem(const void *p, int64_t i, int is_bf16) {
  if (is_bf16) {
    uint32_t u = ((uint32_t)((const uint16_t *)p)[i]) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  return (double)((const float *)p)[i];
}

/* Sequence that owns global row t (cu is non-decreasing). */
static int seq_of_row(const int32_t *cu, int S, int64_t t) {
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  /* skip empty sequences that start at the same offset */
  while (lo + 1 < S && (int64_t)cu[lo + 1] <= t) lo++;
  return lo;
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* Number of blocks of each sequence, and the first global block index of each
 * sequence: first[s] = sum_{s'<s} ceil(L_s'/B), first[S] = total. */
int64_t oracle_block_first(const int32_t *cu, int S, int B, int64_t *first) {
  int64_t acc = 0;
  for (int s = 0; s < S; ++s) {
    if (first) first[s] = acc;
    acc += ceil_div((int64_t)cu[s + 1] - cu[s], B);
  }
  if (first) first[S] = acc;
  return acc;
}

/* [S] "Affinity Scoring": the block representative is the mean of the block's
 * key vectors (over the rows it actually has).
 * kbar: [total_blocks][Hkv][d], global block index = first[s] + j. */
void oracle_meanpool(const void *k, int is_bf16, int64_t T, int Hkv, int d,
                     const int32_t *cu, int S, int B, double *kbar) {
  (void)T;
  int64_t *first = (int64_t *)malloc(sizeof(int64_t) * (S + 1));
  oracle_block_first(cu, S, B, first);
  for (int s = 0; s < S; ++s) {
    int64_t a = cu[s], L = (int64_t)cu[s + 1] - cu[s];
    int64_t nb = ceil_div(L, B);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t j = 0; j < nb; ++j) {
      int64_t r0 = j * B, r1 = (j + 1) * B < L ? (j + 1) * B : L;
      for (int g = 0; g < Hkv; ++g) {
        double *dst = kbar + ((first[s] + j) * Hkv + g) * (int64_t)d;
        for (int e = 0; e < d; ++e) dst[e] = 0.0;
        for (int64_t r = r0; r < r1; ++r)
          for (int e = 0; e < d; ++e)
            dst[e] += load_elem(k, ((a + r) * Hkv + g) * (int64_t)d + e, is_bf16);
        for (int e = 0; e < d; ++e) dst[e] /= (double)(r1 - r0);
      }
    }
  }
  free(first);
}

typedef struct { double s; int j; } cand_t;

/* Order used by the top-k gate: higher score first, then lower block index. */
static int cand_cmp(const void *pa, const void *pb) {
  const cand_t *a = (const cand_t *)pa, *b = (const cand_t *)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->j > b->j) - (a->j < b->j);
}

/* Block selection for a list of query rows (all heads).
 * [S] "Affinity Scoring" (s_i = <q, meanpool(K[I_i])>), "Top-k Gating" (g_i,
 * shared-expert current block), "Causality Enforcement" mechanism 1 (future
 * blocks get -inf); [R] rebuttal W1: every query head selects its own blocks.
 *
 * rows: global row indices (NULL = all T rows in order), n_rows entries.
 * sel: [n_rows][Hq][topk] local block ids, ascending, -1 padded.
 * near_tie: [n_rows][Hq], 1 when the k-th and (k+1)-th ranked gate scores
 *   (the (k-1)-th and k-th ranked historical scores, the current block being
 *   rank 1) differ by less than 1e-3 relative to the larger magnitude.
 * scores: optional [n_rows][Hq][max_blocks] raw scores of candidate blocks
 *   j < c, NAN elsewhere. */
void oracle_select(const void *q, int is_bf16, const double *kbar, int64_t T,
                   int Hq, int Hkv, int d, const int32_t *cu, int S, int B,
                   int topk, const int64_t *rows, int64_t n_rows, int32_t *sel,
                   uint8_t *near_tie, double *scores, int max_blocks) {
  int64_t *first = (int64_t *)malloc(sizeof(int64_t) * (S + 1));
  oracle_block_first(cu, S, B, first);
  int G = Hq / Hkv;
  if (!rows) n_rows = T;
#pragma omp parallel
  {
    cand_t *cand = NULL;
    int64_t cap = 0;
#pragma omp for schedule(dynamic, 64)
    for (int64_t rh = 0; rh < n_rows * Hq; ++rh) {
      int64_t ri = rh / Hq;
      int h = (int)(rh % Hq);
      int64_t t = rows ? rows[ri] : ri;
      int s = seq_of_row(cu, S, t);
      int64_t local = t - cu[s];
      int c = (int)(local / B);            /* current block */
      int g = h / G;                       /* kv head of this query head */
      if (c > cap) { free(cand); cap = c + 64; cand = (cand_t *)malloc(sizeof(cand_t) * cap); }
      /* scores of all earlier blocks; later blocks are never candidates */
      for (int j = 0; j < c; ++j) {
        const double *kb = kbar + ((first[s] + j) * Hkv + g) * (int64_t)d;
        double acc = 0.0;
        for (int e = 0; e < d; ++e)
          acc += load_elem(q, (t * Hq + h) * (int64_t)d + e, is_bf16) * kb[e];
        cand[j].s = acc;
        cand[j].j = j;
      }
      if (scores) {
        double *dst = scores + rh * (int64_t)max_blocks;
        for (int j = 0; j < max_blocks; ++j) dst[j] = NAN;
        for (int j = 0; j < c && j < max_blocks; ++j) dst[j] = cand[j].s;
      }
      if (c > 0) qsort(cand, (size_t)c, sizeof(cand_t), cand_cmp);  /* no candidates: nothing to sort */
      int n_hist = topk - 1 < c ? topk - 1 : c;  /* the current block takes one of the k */
      uint8_t flag = 0;
      if (topk - 1 >= 1 && c > topk - 1) {
        double a = cand[topk - 2].s, b = cand[topk - 1].s;
        double m = fabs(a) > fabs(b) ? fabs(a) : fabs(b);
        flag = fabs(a - b) < 1e-3 * m;
      }
      if (near_tie) near_tie[rh] = flag;
      /* emit ascending: chosen earlier blocks sorted by index, then c */
      int32_t *out = sel + rh * (int64_t)topk;
      int n = 0;
      for (int j = 0; j < c && n < n_hist; ++j) {
        int chosen = 0;
        for (int r = 0; r < n_hist; ++r) chosen |= (cand[r].j == j);
        if (chosen) out[n++] = j;
      }
      out[n++] = c;
      while (n < topk) out[n++] = -1;
    }
    free(cand);
  }
  free(first);
}

/* Fixed gates: sliding window and attention sink.
 * [S] section 3.4 "Context Partitioning": a sliding window is MoBA with a gate
 * that always picks the most recent blocks, an attention sink one that always
 * picks the initial and the recent blocks.
 * Reading: the topk slots hold the n_sink initial blocks (0 <= n_sink < topk)
 * and the topk - n_sink most recent blocks up to and including the current
 * block c; a row with at most topk blocks so far takes all of them. The
 * selection is the same for every head.
 * sel: [n_rows][Hq][topk], ascending, -1 padded. */
void oracle_select_window(const int32_t *cu, int S, int B, int64_t T, int Hq, int topk,
                          int n_sink, const int64_t *rows, int64_t n_rows, int32_t *sel) {
  if (!rows) n_rows = T;
  int w = topk - n_sink;  /* recent blocks, the current one included */
  for (int64_t ri = 0; ri < n_rows; ++ri) {
    int64_t t = rows ? rows[ri] : ri;
    int s = seq_of_row(cu, S, t);
    int c = (int)((t - cu[s]) / B);
    for (int h = 0; h < Hq; ++h) {
      int32_t *out = sel + (ri * Hq + h) * (int64_t)topk;
      int n = 0;
      for (int j = 0; j <= c; ++j)
        if (j < n_sink || j > c - w) out[n++] = j;
      while (n < topk) out[n++] = -1;
    }
  }
}

/* Max- and min-pooled keys: elementwise max / min over the block's rows.
 * [R] authors' rebuttals (W1, on mean pooling / on QUEST): blocks chosen by
 * max-pooled and min-pooled keys on top of the mean-pooled ranking. */
void oracle_minmaxpool(const void *k, int is_bf16, int64_t T, int Hkv, int d,
                       const int32_t *cu, int S, int B, double *kmax, double *kmin) {
  (void)T;
  int64_t *first = (int64_t *)malloc(sizeof(int64_t) * (S + 1));
  oracle_block_first(cu, S, B, first);
  for (int s = 0; s < S; ++s) {
    int64_t a = cu[s], L = (int64_t)cu[s + 1] - cu[s];
    int64_t nb = ceil_div(L, B);
    for (int64_t j = 0; j < nb; ++j) {
      int64_t r0 = j * B, r1 = (j + 1) * B < L ? (j + 1) * B : L;
      for (int g = 0; g < Hkv; ++g) {
        double *mx = kmax + ((first[s] + j) * Hkv + g) * (int64_t)d;
        double *mn = kmin + ((first[s] + j) * Hkv + g) * (int64_t)d;
        for (int e = 0; e < d; ++e) { mx[e] = -INFINITY; mn[e] = INFINITY; }
        for (int64_t r = r0; r < r1; ++r)
          for (int e = 0; e < d; ++e) {
            double x = load_elem(k, ((a + r) * Hkv + g) * (int64_t)d + e, is_bf16);
            if (x > mx[e]) mx[e] = x;
            if (x < mn[e]) mn[e] = x;
          }
      }
    }
  }
  free(first);
}

/* Scores of earlier blocks 0..c-1 against one pooled-key table, sorted by
 * (score desc, index asc); returns 1 when the pick-th and (pick+1)-th scores
 * are a near tie (1e-3 relative), as for the mean gate. */
static int rank_blocks(const void *q, int is_bf16, const double *pool, int64_t t, int Hq, int h,
                       int Hkv, int g, int d, int64_t first, int c, int pick, cand_t *cand) {
  for (int j = 0; j < c; ++j) {
    const double *kb = pool + ((first + j) * Hkv + g) * (int64_t)d;
    double acc = 0.0;
    for (int e = 0; e < d; ++e) acc += load_elem(q, (t * Hq + h) * (int64_t)d + e, is_bf16) * kb[e];
    cand[j].s = acc;
    cand[j].j = j;
  }
  if (c > 0) qsort(cand, (size_t)c, sizeof(cand_t), cand_cmp);
  if (pick < 1 || c <= pick) return 0;
  double a = cand[pick - 1].s, b = cand[pick].s;
  double m = fabs(a) > fabs(b) ? fabs(a) : fabs(b);
  return fabs(a - b) < 1e-3 * m;
}

/* Gate with extra blocks from max- and min-pooled keys.
 * [R] authors' rebuttals: besides the blocks chosen by the mean-pooled gate,
 * the top blocks by max pooling and by min pooling are selected as well.
 * Reading: with W = topk slots, the mean-pooled gate keeps its own-block rule
 * and picks W - extra_max - extra_min - 1 earlier blocks; the max-pooled and
 * min-pooled rankings (raw inner products, same order and tie rule) add their
 * best extra_max and extra_min earlier blocks; the selection is the union.
 * Layout per (row, head): the union's earlier blocks ascending, then -1 for
 * the slots a coinciding pick left empty, then the own block at position
 * min(W, c+1) - 1, then -1. near_tie: any of the three rankings has a near
 * tie at its boundary. */
void oracle_select_pooled(const void *q, int is_bf16, const double *kbar, const double *kmax,
                          const double *kmin, int64_t T, int Hq, int Hkv, int d,
                          const int32_t *cu, int S, int B, int topk, int extra_max,
                          int extra_min, const int64_t *rows, int64_t n_rows, int32_t *sel,
                          uint8_t *near_tie) {
  int64_t *first = (int64_t *)malloc(sizeof(int64_t) * (S + 1));
  oracle_block_first(cu, S, B, first);
  int G = Hq / Hkv;
  if (!rows) n_rows = T;
  int pick_mean = topk - extra_max - extra_min - 1;
#pragma omp parallel
  {
    cand_t *cand = NULL;
    uint8_t *in = NULL;
    int64_t cap = 0;
#pragma omp for schedule(dynamic, 64)
    for (int64_t rh = 0; rh < n_rows * Hq; ++rh) {
      int64_t ri = rh / Hq;
      int h = (int)(rh % Hq);
      int64_t t = rows ? rows[ri] : ri;
      int s = seq_of_row(cu, S, t);
      int c = (int)((t - cu[s]) / B);
      int g = h / G;
      if (c + 1 > cap) {
        free(cand); free(in);
        cap = c + 64;
        cand = (cand_t *)malloc(sizeof(cand_t) * cap);
        in = (uint8_t *)malloc((size_t)cap);
      }
      memset(in, 0, (size_t)c + 1);
      const double *pools[3] = {kbar, kmax, kmin};
      int picks[3] = {pick_mean, extra_max, extra_min};
      uint8_t flag = 0;
      for (int p = 0; p < 3; ++p) {
        flag |= (uint8_t)rank_blocks(q, is_bf16, pools[p], t, Hq, h, Hkv, g, d, first[s], c,
                                     picks[p], cand);
        for (int r = 0; r < picks[p] && r < c; ++r) in[cand[r].j] = 1;
      }
      if (near_tie) near_tie[rh] = flag;
      int32_t *out = sel + rh * (int64_t)topk;
      int nsel = topk < c + 1 ? topk : c + 1;
      int n = 0;
      for (int j = 0; j < c; ++j)
        if (in[j]) out[n++] = j;
      while (n < nsel - 1) out[n++] = -1;
      out[n++] = c;
      while (n < topk) out[n++] = -1;
    }
    free(cand); free(in);
  }
  free(first);
}

/* Attention of one query row over an explicit key-row set.
 * [S] "The Core MoBA Attention Equation": Softmax(q K[I]^T) V[I], with the
 * caller's logit scale; lse = log sum_u exp(z_u). */
static void attend_rows(const void *q, const void *k, const void *v, int is_bf16,
                        int Hq, int Hkv, int d, int64_t t, int h, int g,
                        const int64_t *keys, int64_t nk, double scale,
                        double *z, double *out, double *lse) {
  double m = -INFINITY;
  for (int64_t i = 0; i < nk; ++i) {
    double acc = 0.0;
    for (int e = 0; e < d; ++e)
      acc += load_elem(q, (t * Hq + h) * (int64_t)d + e, is_bf16) *
             load_elem(k, (keys[i] * Hkv + g) * (int64_t)d + e, is_bf16);
    z[i] = scale * acc;
    if (z[i] > m) m = z[i];
  }
  double l = 0.0;
  for (int e = 0; e < d; ++e) out[e] = 0.0;
  for (int64_t i = 0; i < nk; ++i) {
    double p = exp(z[i] - m);
    l += p;
    for (int e = 0; e < d; ++e)
      out[e] += p * load_elem(v, (keys[i] * Hkv + g) * (int64_t)d + e, is_bf16);
  }
  for (int e = 0; e < d; ++e) out[e] /= l;
  *lse = m + log(l);
}

/* Attention over the union of the selected blocks.
 * [S] "Top-k Gating" (I = union of selected blocks), "Causality Enforcement"
 * mechanism 2 (causal mask inside the current block, none in earlier blocks);
 * [C] "Key math / How it works".
 * sel: [n_rows][Hq][topk] local block ids as produced by oracle_select (or any
 * other selection that contains the current block and no later block).
 * out: [n_rows][Hq][d], lse: [n_rows][Hq]. */
void oracle_attend(const void *q, const void *k, const void *v, int is_bf16,
                   int64_t T, int Hq, int Hkv, int d, const int32_t *cu, int S,
                   int B, int topk, const int32_t *sel, const int64_t *rows,
                   int64_t n_rows, double scale, double *out, double *lse) {
  int G = Hq / Hkv;
  if (!rows) n_rows = T;
#pragma omp parallel
  {
    int64_t cap = 0;
    int64_t *keys = NULL;
    double *z = NULL;
#pragma omp for schedule(dynamic, 16)
    for (int64_t rh = 0; rh < n_rows * Hq; ++rh) {
      int64_t ri = rh / Hq;
      int h = (int)(rh % Hq);
      int64_t t = rows ? rows[ri] : ri;
      int s = seq_of_row(cu, S, t);
      int64_t a = cu[s], L = (int64_t)cu[s + 1] - cu[s], local = t - a;
      int64_t c = local / B;
      const int32_t *my = sel + rh * (int64_t)topk;
      int64_t need = (int64_t)topk * B + 1;
      if (need > cap) {
        free(keys); free(z);
        cap = need;
        keys = (int64_t *)malloc(sizeof(int64_t) * cap);
        z = (double *)malloc(sizeof(double) * cap);
      }
      int64_t nk = 0;
      for (int i = 0; i < topk; ++i) {
        int64_t j = my[i];
        if (j < 0) continue;
        int64_t r0 = j * B;
        int64_t r1 = (j == c) ? local + 1 : ((j + 1) * B < L ? (j + 1) * B : L);
        for (int64_t r = r0; r < r1; ++r) keys[nk++] = a + r;
      }
      attend_rows(q, k, v, is_bf16, Hq, Hkv, d, t, h, h / G, keys, nk, scale, z,
                  out + rh * (int64_t)d, lse + rh);
    }
    free(keys); free(z);
  }
}

/* Gradients of the block-sparse attention for a given selection.
 * [S] section 3.4 and [C] "Key math": the output of (t, h) is
 * softmax(scale * q K[I]^T) V[I] over the union I of its selected blocks
 * (own block causally); the selection is a discrete choice, so gradients
 * flow through this attention only (the gate receives none).
 * With P_u = exp(z_u - lse), z_u = scale <q, k_u>, for every (t, h):
 *   dV[u] += P_u dO,  dP_u = <dO, v_u>,  D = sum_u P_u dP_u,
 *   dS_u = P_u (dP_u - D),  dQ = scale sum_u dS_u k_u,  dK[u] += scale dS_u q.
 * All rows t of the tensors take part (no row subset). dq [T][Hq][d],
 * dk and dv [T][Hkv][d] (double, zeroed here). */
void oracle_attend_bwd(const void *q, const void *k, const void *v, const double *dout,
                       int is_bf16, int64_t T, int Hq, int Hkv, int d, const int32_t *cu, int S,
                       int B, int topk, const int32_t *sel, double scale, double *dq, double *dk,
                       double *dv) {
  const int G = Hq / Hkv;
  memset(dq, 0, sizeof(double) * (size_t)T * Hq * d);
  memset(dk, 0, sizeof(double) * (size_t)T * Hkv * d);
  memset(dv, 0, sizeof(double) * (size_t)T * Hkv * d);
  int64_t cap = (int64_t)topk * B + 1;
  /* kv heads are independent (each owns its query heads' rows of dq and its
   * own dk, dv); inside one, rows and heads run in order */
#pragma omp parallel for schedule(static, 1)
  for (int g = 0; g < Hkv; ++g) {
    int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * cap);
    double *z = (double *)malloc(sizeof(double) * cap);
    double *dp = (double *)malloc(sizeof(double) * cap);
    for (int64_t t = 0; t < T; ++t) {
      int s = seq_of_row(cu, S, t);
      int64_t a = cu[s], L = (int64_t)cu[s + 1] - cu[s], local = t - a, c = local / B;
      for (int h = g * G; h < (g + 1) * G; ++h) {
        const int32_t *my = sel + (t * Hq + h) * (int64_t)topk;
        int64_t nk = 0;
        for (int i = 0; i < topk; ++i) {
          int64_t j = my[i];
          if (j < 0) continue;
          int64_t r0 = j * B, r1 = (j == c) ? local + 1 : ((j + 1) * B < L ? (j + 1) * B : L);
          for (int64_t r = r0; r < r1; ++r) keys[nk++] = a + r;
        }
        double m = -INFINITY;
        for (int64_t i = 0; i < nk; ++i) {
          double acc = 0.0;
          for (int e = 0; e < d; ++e)
            acc += load_elem(q, (t * Hq + h) * (int64_t)d + e, is_bf16) *
                   load_elem(k, (keys[i] * Hkv + g) * (int64_t)d + e, is_bf16);
          z[i] = scale * acc;
          if (z[i] > m) m = z[i];
        }
        double l = 0.0;
        for (int64_t i = 0; i < nk; ++i) { z[i] = exp(z[i] - m); l += z[i]; }
        const double *go = dout + (t * Hq + h) * (int64_t)d;
        double D = 0.0;
        for (int64_t i = 0; i < nk; ++i) {
          z[i] /= l;  /* P_u */
          double acc = 0.0;
          for (int e = 0; e < d; ++e)
            acc += go[e] * load_elem(v, (keys[i] * Hkv + g) * (int64_t)d + e, is_bf16);
          dp[i] = acc;
          D += z[i] * acc;
        }
        double *gq = dq + (t * Hq + h) * (int64_t)d;
        for (int64_t i = 0; i < nk; ++i) {
          double ds = z[i] * (dp[i] - D);
          double *gk = dk + (keys[i] * Hkv + g) * (int64_t)d;
          double *gv = dv + (keys[i] * Hkv + g) * (int64_t)d;
          for (int e = 0; e < d; ++e) {
            gq[e] += scale * ds * load_elem(k, (keys[i] * Hkv + g) * (int64_t)d + e, is_bf16);
            gk[e] += scale * ds * load_elem(q, (t * Hq + h) * (int64_t)d + e, is_bf16);
            gv[e] += z[i] * go[e];
          }
        }
      }
    }
    free(keys); free(z); free(dp);
  }
}

/* dq alone for a list of rows (all heads): the query-side half of
 * oracle_attend_bwd, in the same order of operations, for sampled rows of
 * inputs too large for the full gradient. sel and dout hold the listed rows:
 * sel [n_rows][Hq][topk], dout [n_rows][Hq][d]; dq [n_rows][Hq][d]. */
void oracle_attend_bwd_dq_rows(const void *q, const void *k, const void *v, const double *dout,
                               int is_bf16, int64_t T, int Hq, int Hkv, int d, const int32_t *cu,
                               int S, int B, int topk, const int32_t *sel, const int64_t *rows,
                               int64_t n_rows, double scale, double *dq) {
  const int G = Hq / Hkv;
  const int64_t cap = (int64_t)topk * B + 1;
  (void)T;
#pragma omp parallel
  {
    int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * cap);
    double *z = (double *)malloc(sizeof(double) * cap);
    double *dp = (double *)malloc(sizeof(double) * cap);
#pragma omp for schedule(dynamic, 1)
    for (int64_t w = 0; w < n_rows * Hq; ++w) {
      const int64_t ri = w / Hq, t = rows[ri];
      const int h = (int)(w % Hq), g = h / G;
      int s = seq_of_row(cu, S, t);
      int64_t a = cu[s], L = (int64_t)cu[s + 1] - cu[s], local = t - a, c = local / B;
      const int32_t *my = sel + (ri * Hq + h) * (int64_t)topk;
      int64_t nk = 0;
      for (int i = 0; i < topk; ++i) {
        int64_t j = my[i];
        if (j < 0) continue;
        int64_t r0 = j * B, r1 = (j == c) ? local + 1 : ((j + 1) * B < L ? (j + 1) * B : L);
        for (int64_t r = r0; r < r1; ++r) keys[nk++] = a + r;
      }
      double m = -INFINITY;
      for (int64_t i = 0; i < nk; ++i) {
        double acc = 0.0;
        for (int e = 0; e < d; ++e)
          acc += load_elem(q, (t * Hq + h) * (int64_t)d + e, is_bf16) *
                 load_elem(k, (keys[i] * Hkv + g) * (int64_t)d + e, is_bf16);
        z[i] = scale * acc;
        if (z[i] > m) m = z[i];
      }
      double l = 0.0;
      for (int64_t i = 0; i < nk; ++i) { z[i] = exp(z[i] - m); l += z[i]; }
      const double *go = dout + (ri * Hq + h) * (int64_t)d;
      double D = 0.0;
      for (int64_t i = 0; i < nk; ++i) {
        z[i] /= l;
        double acc = 0.0;
        for (int e = 0; e < d; ++e)
          acc += go[e] * load_elem(v, (keys[i] * Hkv + g) * (int64_t)d + e, is_bf16);
        dp[i] = acc;
        D += z[i] * acc;
      }
      double *gq = dq + (ri * Hq + h) * (int64_t)d;
      for (int e = 0; e < d; ++e) gq[e] = 0.0;
      for (int64_t i = 0; i < nk; ++i) {
        double ds = z[i] * (dp[i] - D);
        for (int e = 0; e < d; ++e)
          gq[e] += scale * ds * load_elem(k, (keys[i] * Hkv + g) * (int64_t)d + e, is_bf16);
      }
    }
    free(keys); free(z); free(dp);
  }
}

/* Full MoBA forward for a list of rows: meanpool, select, attend.
 * sel_out / near_tie_out may be NULL. */
void oracle_moba(const void *q, const void *k, const void *v, int is_bf16,
                 int64_t T, int Hq, int Hkv, int d, const int32_t *cu, int S,
                 int B, int topk, double scale, const int64_t *rows,
                 int64_t n_rows, double *out, double *lse, int32_t *sel_out,
                 uint8_t *near_tie_out) {
  int64_t nb = oracle_block_first(cu, S, B, NULL);
  double *kbar = (double *)malloc(sizeof(double) * (nb > 0 ? nb : 1) * Hkv * d);
  oracle_meanpool(k, is_bf16, T, Hkv, d, cu, S, B, kbar);
  int64_t nr = rows ? n_rows : T;
  int32_t *sel = sel_out ? sel_out : (int32_t *)malloc(sizeof(int32_t) * (nr > 0 ? nr : 1) * Hq * topk);
  oracle_select(q, is_bf16, kbar, T, Hq, Hkv, d, cu, S, B, topk, rows, nr, sel,
                near_tie_out, NULL, 0);
  oracle_attend(q, k, v, is_bf16, T, Hq, Hkv, d, cu, S, B, topk, sel, rows, nr,
                scale, out, lse);
  if (!sel_out) free(sel);
  free(kbar);
}

/* Dense causal attention (the full-attention baseline the pages compare to):
 * [S] "Standard Attention Baseline" with the usual causal mask, per sequence. */
void oracle_dense_causal(const void *q, const void *k, const void *v, int is_bf16,
                         int64_t T, int Hq, int Hkv, int d, const int32_t *cu,
                         int S, const int64_t *rows, int64_t n_rows, double scale,
                         double *out, double *lse) {
  int G = Hq / Hkv;
  if (!rows) n_rows = T;
#pragma omp parallel
  {
    int64_t cap = 0;
    int64_t *keys = NULL;
    double *z = NULL;
#pragma omp for schedule(dynamic, 16)
    for (int64_t rh = 0; rh < n_rows * Hq; ++rh) {
      int64_t ri = rh / Hq;
      int h = (int)(rh % Hq);
      int64_t t = rows ? rows[ri] : ri;
      int s = seq_of_row(cu, S, t);
      int64_t a = cu[s], nk = t - a + 1;
      if (nk > cap) {
        free(keys); free(z);
        cap = nk;
        keys = (int64_t *)malloc(sizeof(int64_t) * cap);
        z = (double *)malloc(sizeof(double) * cap);
      }
      for (int64_t i = 0; i < nk; ++i) keys[i] = a + i;
      attend_rows(q, k, v, is_bf16, Hq, Hkv, d, t, h, h / G, keys, nk, scale, z,
                  out + rh * (int64_t)d, lse + rh);
    }
    free(keys); free(z);
  }
}
