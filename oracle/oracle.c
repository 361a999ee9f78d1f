/*
 * oracle.c -- plain, slow CPU reference for block-sparse causal prefill attention.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the package's smoke check and the benchmark's
 * CPU-baseline leg load this library.  The product path never calls it, and it shares no
 * code, header, table or helper with the GPU library.
 *
 * What it computes, step by step, and where each step is defined:
 *
 *   1. Block summaries.  "Uncertainty-Gated Selection for Block-Sparse Attention" page,
 *      Metodologia step 1: keys are grouped in blocks and scored by an existing backbone,
 *      either the SSA-style mean-pooled key or Quest's per-coordinate K-min/K-max upper
 *      bound.  The Stem page (Metodologia B, the output-aware metric) adds the value
 *      magnitude; the product form used here multiplies the tile score by the mean over the
 *      block's rows of each value row's L2 norm.
 *   2. Tile scores.  Same page, step 2: selection is per query tile; a block's tile score
 *      is the maximum over the tile's query rows.
 *   3. Budget.  Stem page, Metodologia A (token position decay): a larger budget for early
 *      positions and a linear decay toward late ones; or a constant k.
 *   4. Ranking and top-k over the free (non-forced) causal blocks.
 *   5. Cut margin.  Same gated-selection page, step 3, the normalised margin
 *      sigma = (s_(k-1) - s_(k)) / (s_(0) - s_(k)) over the sorted scores.
 *   6. Head mean and gate.  Step 4: sigma averaged over heads, tripped when it falls to or
 *      below a per-layer empirical quantile q.
 *   7. Expansion and padding.  Step 5: tripped tiles keep the top floor(rho*k) blocks,
 *      the others k; lists are padded with sentinels to one uniform width.
 *   8. Attention.  Exact softmax attention of each query row over the keys of its selected
 *      blocks, causally masked (the pages' FlashAttention-style pass computes exactly this;
 *      online softmax is order-invariant, ART page section 2.4).
 *
 * Precision.  The pages fix no precision.  Steps 1-7 decide integers (which blocks are
 * kept, which tiles trip), so they run in the same IEEE fp32 arithmetic the GPU kernels
 * use, with every operation and its order written out below (the canonical arithmetic);
 * this is what makes selections comparable bit for bit.  Step 8 has a plain definition
 * and is computed in fp64.
 *
 * Canonical fp32 arithmetic (compile with -ffp-contract=off; fmaf is a fused multiply-add):
 *   - bf16 -> fp32 conversion is exact; every accumulator starts at +0.0f and runs in
 *     index order; canon(x) = x + 0.0f maps -0 to +0 and nothing else.
 *   - kmean_c = (sum over rows r in order of k_rc) * (1/block)   (block is a power of two)
 *   - kmin_c = canon(min_r k_rc), kmax_c = canon(max_r k_rc)
 *   - vnorm = (sum over rows r in order of sqrtf(ss_r)) * (1/block),
 *             ss_r = fmaf chain over c in order of v_rc * v_rc
 *   - row score s_ij = fmaf chain over c in order of q_ic * x_jc, where x = kmean, or for
 *     the bound x_c = (q_ic >= 0 ? kmax_c : kmin_c); no 1/sqrt(d) (ranking and sigma are
 *     invariant to a positive scale)
 *   - tile score S_tj = canon(max over the tile's rows of s_ij); output-aware, product form
 *     (output_aware = 1): S_tj = canon(S_tj * vnorm_j); additive form (output_aware = 2,
 *     Stem page, Metodologia B: score plus beta * max(0, log ||V_j||^2)):
 *     S_tj = canon(fmaf(S_tj, scale, bonus_j)), scale = (float)(1 / sqrt(d)) puts the score
 *     on the logit scale, bonus_j = (float)(beta * max(0, ln(vnorm_j^2))) with the logarithm,
 *     the square and the product taken in fp64
 *   - sigma: two fp32 subtractions and one IEEE division; sigma_bar: fp32 sum over heads in
 *     order, divided by the head count; the quantile rank ceil(q*M) in fp64.
 *
 * Readings where the pages leave a step open (each is listed in the design notes):
 *   - Forced blocks (the diagonal, and the first n_sink blocks) are kept on top of k and
 *     take no part in ranking or sigma; k counts free picks only.
 *   - Ranking key: score descending, then block index ascending.
 *   - A tile with at most k free candidates is not eligible: sigma is reported as 1, it
 *     never trips, it is left out of the quantile, and all its free blocks are kept.
 *   - sigma = 0 when s_(0) == s_(k).
 *   - Quantile: tau_b is the ceil(q*M_b)-th smallest sigma_bar over batch element b's
 *     eligible tiles (inverted empirical CDF); a tile trips iff eligible and
 *     sigma_bar <= tau_b; ceil(q*M) = 0 trips nothing (tau reported as -inf).
 *   - Budget linear decay: k_t = max(k_min, floor(k_max * (n - t) / n)) in integers.
 *   - Lists are ascending block indices padded with -1; a count array comes with them.
 *   - Tile != block: tile t's diagonal blocks are all blocks overlapping its rows (forced);
 *     its free blocks are the earlier ones; the budget's position decay runs over tiles.
 *   - Group-shared selection (select_unit = 1; not on the pages, which select per query
 *     head): one list per kv head, the tile score being the maximum over the tile's rows of
 *     all that kv head's query heads; sigma per kv head, sigma_bar their mean.
 */

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Problem description, mirrored field for field by a ctypes Structure in __init__.py. */
typedef struct {
  int32_t batch, seqlen, n_q_heads, n_kv_heads, head_dim, block; /* block: keys per block */
  int32_t in_dtype;     /* 0: float32 arrays, 1: bfloat16 bit patterns (uint16) */
  int32_t score_mode;   /* 0: mean-pooled keys, 1: per-coordinate min/max bound */
  int32_t output_aware; /* 1: tile score times mean value-row L2 norm; 2: additive form */
  int32_t k_max, k_min, budget_kind; /* budget_kind 0: constant k_max, 1: linear decay */
  int32_t n_sink;       /* first n_sink blocks are always kept */
  int32_t gate_mode;    /* 0: per-call quantile, 1: fixed threshold, 2: no gate */
  float tau_fixed;
  float oam_beta;       /* beta of the additive output-aware form */
  double rho, q;
  int32_t width;        /* entries per padded list */
  int32_t select_unit;  /* 0: one list per query head; 1: one list per kv head, shared by its
                           query heads (see tile_score) */
  int32_t tile;         /* query tile rows T (0: equal to block); a multiple of block, or a
                           divisor of it */
  int32_t pad3_;
} oc_cfg;

/* ---------------------------------------------------------------- element access */

static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static float elem(const void* p, int dtype, int64_t i) {
  if (dtype == 0) return ((const float*)p)[i];
  return bf16_to_f32(((const uint16_t*)p)[i]);
}

static float canon(float x) { return x + 0.0f; }

/* Index of element (b, pos, head, c) in a contiguous [B, N, H, d] tensor. */
static int64_t bshd(const oc_cfg* c, int b, int64_t pos, int head, int nheads, int ch) {
  return (((int64_t)b * c->seqlen + pos) * nheads + head) * c->head_dim + ch;
}

/* Index of summary element (b, block j, kv head g, coordinate ch) in [B, n, Hkv, d]. */
static int64_t sidx(const oc_cfg* c, int b, int j, int g, int ch) {
  int n = c->seqlen / c->block;
  return (((int64_t)b * n + j) * c->n_kv_heads + g) * c->head_dim + ch;
}

/* ------------------------------------------------------------- 1. block summaries */

/* K [B,N,Hkv,d] (and V when output-aware) -> kA [B,n,Hkv,d] (kmean, or kmin), kB (kmax,
 * bound mode only), vn [B,n,Hkv] (output-aware only). */
int oracle_pool(const oc_cfg* c, const void* K, const void* V, float* kA, float* kB,
                float* vn) {
  const int n = c->seqlen / c->block, d = c->head_dim, Hkv = c->n_kv_heads;
  const float inv_blk = 1.0f / (float)c->block;
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < c->batch; ++b)
    for (int j = 0; j < n; ++j)
      for (int g = 0; g < Hkv; ++g) {
        for (int ch = 0; ch < d; ++ch) {
          if (c->score_mode == 0) {
            float acc = 0.0f;
            for (int r = 0; r < c->block; ++r)
              acc = acc + elem(K, c->in_dtype, bshd(c, b, (int64_t)j * c->block + r, g, Hkv, ch));
            kA[sidx(c, b, j, g, ch)] = acc * inv_blk;
          } else {
            float lo = elem(K, c->in_dtype, bshd(c, b, (int64_t)j * c->block, g, Hkv, ch));
            float hi = lo;
            for (int r = 1; r < c->block; ++r) {
              float x = elem(K, c->in_dtype, bshd(c, b, (int64_t)j * c->block + r, g, Hkv, ch));
              if (x < lo) lo = x;
              if (x > hi) hi = x;
            }
            kA[sidx(c, b, j, g, ch)] = canon(lo);
            kB[sidx(c, b, j, g, ch)] = canon(hi);
          }
        }
        if (c->output_aware) {
          float acc = 0.0f;
          for (int r = 0; r < c->block; ++r) {
            float ss = 0.0f;
            for (int ch = 0; ch < d; ++ch) {
              float v = elem(V, c->in_dtype, bshd(c, b, (int64_t)j * c->block + r, g, Hkv, ch));
              ss = fmaf(v, v, ss);
            }
            acc = acc + sqrtf(ss);
          }
          vn[((int64_t)b * n + j) * Hkv + g] = acc * inv_blk;
        }
      }
  return 0;
}

/* ---------------------------------------------------------------- 2. tile scores */

/* Query tiles.  The pages' tile is a query block scored against key blocks (gated-selection
 * page, Metodologia step 2); the workloads have tile = block.  A tile of T rows over blocks
 * of blk keys reads as: tile t holds rows tT .. tT+T-1; its causal blocks are those starting
 * at or before its last row, j < diag_end(t); the blocks overlapping its rows,
 * diag_first(t) <= j < diag_end(t), are its diagonal blocks (forced, as the single diagonal
 * block is when T = blk). */
static int tile_rows(const oc_cfg* c) { return c->tile > 0 ? c->tile : c->block; }
static int n_tiles(const oc_cfg* c) { return c->seqlen / tile_rows(c); }
static int diag_first(const oc_cfg* c, int t) {
  return (int)((int64_t)t * tile_rows(c) / c->block);
}
static int diag_end(const oc_cfg* c, int t) {
  return (int)(((int64_t)(t + 1) * tile_rows(c) - 1) / c->block) + 1;
}

/* Selection units.  The gated-selection page selects per query tile and head (Metodologia
 * steps 2-3), one list per query head.  Its GQA form with one list per kv head, shared by that
 * kv head's G query heads, is not on the pages; this oracle reads it as the same algorithm
 * run on "the query rows of the tile in all G heads": the tile score of step 2 is the maximum
 * of the row scores over those G x tile rows, and steps 3-5 then run per kv head exactly as
 * they run per query head, sigma_bar averaging over the kv heads. */
static int units(const oc_cfg* c) { return c->select_unit ? c->n_kv_heads : c->n_q_heads; }
static int heads_per_unit(const oc_cfg* c) {
  return c->select_unit ? c->n_q_heads / c->n_kv_heads : 1;
}

typedef struct {
  const oc_cfg* c;
  const void* Q;
  const float *kA, *kB, *vn;
} oc_inputs;

/* Raw fp32 score of query row (b, pos, h) against block j's summary. */
static float row_score(const oc_inputs* in, int b, int64_t pos, int h, int j) {
  const oc_cfg* c = in->c;
  const int g = h / (c->n_q_heads / c->n_kv_heads);
  float s = 0.0f;
  for (int ch = 0; ch < c->head_dim; ++ch) {
    float q = elem(in->Q, c->in_dtype, bshd(c, b, pos, h, c->n_q_heads, ch));
    float x;
    if (c->score_mode == 0)
      x = in->kA[sidx(c, b, j, g, ch)];
    else
      x = (q >= 0.0f) ? in->kB[sidx(c, b, j, g, ch)] : in->kA[sidx(c, b, j, g, ch)];
    s = fmaf(q, x, s);
  }
  return s;
}

/* Additive output-aware term of block j (Stem page, Metodologia B): beta times the positive
 * part of the natural log of the squared value norm, in fp64, rounded once to fp32. */
static float oam_bonus(float vnorm, float beta) {
  const double l = log((double)vnorm * (double)vnorm);
  return (float)((double)beta * (l > 0.0 ? l : 0.0));
}

/* Tile score S_tj of selection unit u: maximum over the tile's rows (of every query head of
 * the unit), then the output-aware factor or term. */
static float tile_score(const oc_inputs* in, int b, int u, int t, int j) {
  const oc_cfg* c = in->c;
  const int gs = heads_per_unit(c), h0 = u * gs, T = tile_rows(c);
  float m = row_score(in, b, (int64_t)t * T, h0, j);
  for (int h = h0; h < h0 + gs; ++h)
    for (int r = 0; r < T; ++r) {
      float s = row_score(in, b, (int64_t)t * T + r, h, j);
      if (s > m) m = s;
    }
  m = canon(m);
  if (c->output_aware) {
    const int n = c->seqlen / c->block;
    const int g = h0 / (c->n_q_heads / c->n_kv_heads);
    const float v = in->vn[((int64_t)b * n + j) * c->n_kv_heads + g];
    if (c->output_aware == 1) {
      m = canon(m * v);
    } else {
      /* the score on the logit scale (1/sqrt(d), as the attention's softmax sees it) */
      const float scale = (float)(1.0 / sqrt((double)c->head_dim));
      m = canon(fmaf(m, scale, oam_bonus(v, c->oam_beta)));
    }
  }
  return m;
}

/* ------------------------------------------------------------ 3. budget and forced set */

/* Budget of tile t: the position decay runs over the tile index (tiles = n_tiles). */
static int budget(const oc_cfg* c, int t) {
  const int n = n_tiles(c);
  if (c->budget_kind == 0) return c->k_max;
  int64_t k = (int64_t)c->k_max * (n - t) / n;
  return k > c->k_min ? (int)k : c->k_min;
}

/* Forced blocks of tile t: its diagonal blocks (every block that overlaps the tile's rows)
 * and the sinks. */
static int is_forced(const oc_cfg* c, int t, int j) {
  return j >= diag_first(c, t) || j < c->n_sink;
}

static int expanded(const oc_cfg* c, int k) { return (int)floor(c->rho * (double)k); }

/* ---------------------------------------------------------------- 4. ranking */

typedef struct {
  float s;
  int j;
} scored;

/* Total order: higher score first, then lower block index. */
static int by_rank(const void* pa, const void* pb) {
  const scored* a = (const scored*)pa;
  const scored* b = (const scored*)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->j < b->j) ? -1 : (a->j > b->j);
}

/* Scores every free causal block of tile t for unit u and ranks them; returns the count. */
static int rank_free(const oc_inputs* in, int b, int u, int t, scored* out) {
  int m = 0;
  for (int j = 0; j < diag_end(in->c, t); ++j) {
    if (is_forced(in->c, t, j)) continue;
    out[m].s = tile_score(in, b, u, t, j);
    out[m].j = j;
    ++m;
  }
  qsort(out, (size_t)m, sizeof(scored), by_rank);
  return m;
}

/* ---------------------------------------------------------------- 5. cut margin */

/* sigma over the ranked free scores; sets *eligible. */
static float cut_margin(const scored* r, int m, int k, int* eligible) {
  if (m <= k) {
    *eligible = 0;
    return 1.0f;
  }
  *eligible = 1;
  float num = r[k - 1].s - r[k].s;
  float den = r[0].s - r[k].s;
  if (den == 0.0f) return 0.0f;
  return num / den;
}

/* ---------------------------------------------------------------- 7. list emission */

static int cmp_int(const void* a, const void* b) {
  int x = *(const int*)a, y = *(const int*)b;
  return (x > y) - (x < y);
}

/* Forced blocks plus the first `keep` ranked free blocks, ascending, -1 padded. */
static int emit_list(const oc_cfg* c, int t, const scored* r, int keep, int* list) {
  int cnt = 0;
  for (int j = 0; j < diag_end(c, t); ++j)
    if (is_forced(c, t, j)) list[cnt++] = j;
  for (int e = 0; e < keep; ++e) list[cnt++] = r[e].j;
  qsort(list, (size_t)cnt, sizeof(int), cmp_int);
  for (int e = cnt; e < c->width; ++e) list[e] = -1;
  return cnt;
}

static int keep_count(const oc_cfg* c, int t, int m, int tripped) {
  int k = budget(c, t);
  int keep = tripped ? expanded(c, k) : k;
  return keep < m ? keep : m;
}

/* ---------------------------------------------------------------- 6. gate */

static int cmp_float(const void* a, const void* b) {
  float x = *(const float*)a, y = *(const float*)b;
  return (x > y) - (x < y);
}

/* Per batch element: tau from the eligible tiles' sigma_bar, and the gate bits. */
static void gate_batch(const oc_cfg* c, const float* sbar, const int* elig, float* tau,
                       unsigned char* gate) {
  const int n = n_tiles(c);
  float t_b = -INFINITY;
  if (c->gate_mode == 0) {
    float* vals = (float*)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
    int M = 0;
    for (int t = 0; t < n; ++t)
      if (elig[t]) vals[M++] = sbar[t];
    double rq = ceil(c->q * (double)M);
    int r = rq < 0 ? 0 : (rq > M ? M : (int)rq);
    if (r > 0) {
      qsort(vals, (size_t)M, sizeof(float), cmp_float);
      t_b = vals[r - 1];
    }
    free(vals);
  } else if (c->gate_mode == 1) {
    t_b = c->tau_fixed;
  }
  *tau = t_b;
  for (int t = 0; t < n; ++t)
    gate[t] = (unsigned char)(c->gate_mode != 2 && elig[t] && sbar[t] <= t_b);
}

/* ------------------------------------------------------- whole selection (steps 2-7) */

/* Q [B,N,Hq,d]; summaries from oracle_pool.  With U selection units (Hq, or Hkv when lists
 * are per kv head) and n = N / T tiles, outputs: kv_idx [B,U,n,W], kv_cnt [B,U,n],
 * sigma [B,U,n], sigma_bar [B,n], gate [B,n], tau [B]. */
int oracle_select(const oc_cfg* c, const void* Q, const float* kA, const float* kB,
                  const float* vn, int32_t* kv_idx, int32_t* kv_cnt, float* sigma,
                  float* sigma_bar, unsigned char* gate, float* tau) {
  const int n = n_tiles(c), Hq = units(c), W = c->width;
  oc_inputs in = {c, Q, kA, kB, vn};
  int Rmax = c->seqlen / c->block; /* ranked entries kept per (b, h, t): all free blocks */
  scored* ranked = (scored*)malloc(sizeof(scored) * (size_t)c->batch * Hq * n * Rmax);
  int* nfree = (int*)malloc(sizeof(int) * (size_t)c->batch * Hq * n);
  int* elig = (int*)malloc(sizeof(int) * (size_t)c->batch * n);
  if (!ranked || !nfree || !elig) return -1;

#pragma omp parallel for collapse(3) schedule(dynamic, 1)
  for (int b = 0; b < c->batch; ++b)
    for (int h = 0; h < Hq; ++h)
      for (int t = 0; t < n; ++t) {
        int64_t bht = ((int64_t)b * Hq + h) * n + t;
        scored* r = ranked + bht * Rmax;
        int m = rank_free(&in, b, h, t, r);
        int e;
        sigma[bht] = cut_margin(r, m, budget(c, t), &e);
        nfree[bht] = m;
        if (h == 0) elig[(int64_t)b * n + t] = e;
      }

  for (int b = 0; b < c->batch; ++b) {
    for (int t = 0; t < n; ++t) {
      float acc = 0.0f; /* over the units: heads, or kv heads */
      for (int h = 0; h < Hq; ++h) acc = acc + sigma[((int64_t)b * Hq + h) * n + t];
      sigma_bar[(int64_t)b * n + t] = acc / (float)Hq;
    }
    gate_batch(c, sigma_bar + (int64_t)b * n, elig + (int64_t)b * n, tau + b,
               gate + (int64_t)b * n);
  }

#pragma omp parallel for collapse(3) schedule(static)
  for (int b = 0; b < c->batch; ++b)
    for (int h = 0; h < Hq; ++h)
      for (int t = 0; t < n; ++t) {
        int64_t bht = ((int64_t)b * Hq + h) * n + t;
        int keep = keep_count(c, t, nfree[bht], gate[(int64_t)b * n + t]);
        kv_cnt[bht] = emit_list(c, t, ranked + bht * Rmax, keep, kv_idx + bht * W);
      }
  free(ranked);
  free(nfree);
  free(elig);
  return 0;
}

/* One tile (b, t) on its own, for checks at sizes where the whole selection is too slow:
 * sigma for every selection unit [U], sigma_bar, eligibility, and for every unit the list
 * emitted if the tile does not trip (lists[0][u][:], cnts[0][u]) and if it does (lists[1],
 * cnts[1]).  The gate itself needs every tile of the batch element and is not computed here. */
int oracle_select_tile(const oc_cfg* c, const void* Q, const float* kA, const float* kB,
                       const float* vn, int b, int t, float* sigma_h, float* sigma_bar,
                       int32_t* eligible, int32_t* lists, int32_t* cnts) {
  const int n = c->seqlen / c->block, Hq = units(c), W = c->width; /* n: blocks */
  oc_inputs in = {c, Q, kA, kB, vn};
  scored* ranked = (scored*)malloc(sizeof(scored) * (size_t)Hq * n);
  int* nfree = (int*)malloc(sizeof(int) * (size_t)Hq);
  int e0 = 0;
  if (!ranked || !nfree) return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int h = 0; h < Hq; ++h) {
    int e;
    nfree[h] = rank_free(&in, b, h, t, ranked + (int64_t)h * n);
    sigma_h[h] = cut_margin(ranked + (int64_t)h * n, nfree[h], budget(c, t), &e);
    if (h == 0) e0 = e;
  }
  float acc = 0.0f;
  for (int h = 0; h < Hq; ++h) acc = acc + sigma_h[h];
  *sigma_bar = acc / (float)Hq;
  *eligible = e0;
  for (int tripped = 0; tripped < 2; ++tripped)
    for (int h = 0; h < Hq; ++h) {
      int keep = keep_count(c, t, nfree[h], tripped);
      cnts[tripped * Hq + h] =
          emit_list(c, t, ranked + (int64_t)h * n, keep, lists + ((int64_t)tripped * Hq + h) * W);
    }
  free(ranked);
  free(nfree);
  (void)n;
  return 0;
}

/* Tile scores of the causal blocks j < diag_end(t) of tile t for selection unit h (forced
 * blocks: NaN); returns diag_end(t). */
int oracle_tile_scores(const oc_cfg* c, const void* Q, const float* kA, const float* kB,
                       const float* vn, int b, int h, int t, float* S) {
  oc_inputs in = {c, Q, kA, kB, vn};
  const int e = diag_end(c, t);
  for (int j = 0; j < e; ++j) S[j] = is_forced(c, t, j) ? NAN : tile_score(&in, b, h, t, j);
  return e;
}

/* Tiles per sequence and the causal-block end of tile t, exported for the tests. */
int oracle_n_tiles(const oc_cfg* c) { return n_tiles(c); }
int oracle_diag_end(const oc_cfg* c, int t) { return diag_end(c, t); }

/* Raw row score s_ij of query position pos against block j (one fmaf chain). */
float oracle_row_score(const oc_cfg* c, const void* Q, const float* kA, const float* kB,
                       int b, int64_t pos, int h, int j) {
  oc_inputs in = {c, Q, kA, kB, NULL};
  return row_score(&in, b, pos, h, j);
}

/* ---------------------------------------------------------------- 8. attention (fp64) */

/* Softmax attention of query row (b, pos, h) over the keys of the listed blocks that are
 * not after pos.  Writes d outputs and the natural-log log-sum-exp of the scaled logits. */
static void attend_row(const oc_cfg* c, const void* Q, const void* K, const void* V,
                       const int32_t* list, int cnt, double scale, int b, int64_t pos, int h,
                       double* out, double* lse, double* z) {
  const int d = c->head_dim, Hq = c->n_q_heads, Hkv = c->n_kv_heads, g = h / (Hq / Hkv);
  int nk = 0;
  double zmax = -INFINITY;
  for (int e = 0; e < cnt; ++e) {
    int j = list[e];
    if (j < 0) break;
    for (int r = 0; r < c->block; ++r) {
      int64_t p = (int64_t)j * c->block + r;
      if (p > pos) continue;
      double dot = 0.0;
      for (int ch = 0; ch < d; ++ch)
        dot += (double)elem(Q, c->in_dtype, bshd(c, b, pos, h, Hq, ch)) *
               (double)elem(K, c->in_dtype, bshd(c, b, p, g, Hkv, ch));
      z[2 * nk] = dot * scale;
      z[2 * nk + 1] = (double)p;
      if (z[2 * nk] > zmax) zmax = z[2 * nk];
      ++nk;
    }
  }
  double den = 0.0;
  for (int ch = 0; ch < d; ++ch) out[ch] = 0.0;
  for (int e = 0; e < nk; ++e) {
    double w = exp(z[2 * e] - zmax);
    int64_t p = (int64_t)z[2 * e + 1];
    den += w;
    for (int ch = 0; ch < d; ++ch) out[ch] += w * (double)elem(V, c->in_dtype, bshd(c, b, p, g, Hkv, ch));
  }
  for (int ch = 0; ch < d; ++ch) out[ch] /= den;
  *lse = zmax + log(den);
}

/* Rows to compute: rows[3*i .. 3*i+2] = (b, h, pos) for i < n_rows; rows == NULL means every
 * row, in [B, N, Hq] order.  O receives n_rows x d doubles, lse n_rows doubles (may be NULL).
 * The list of row (b, h, pos) is kv_idx[b, u, pos / T, :], with kv_cnt entries, for the
 * selection unit u of head h (h itself, or its kv head). */
int oracle_forward(const oc_cfg* c, const void* Q, const void* K, const void* V,
                   const int32_t* kv_idx, const int32_t* kv_cnt, int W, float softmax_scale,
                   int64_t n_rows, const int64_t* rows, double* O, double* lse) {
  const int n = n_tiles(c), Hq = c->n_q_heads, d = c->head_dim;
  if (rows == NULL) n_rows = (int64_t)c->batch * c->seqlen * Hq;
  int fail = 0;
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * 2 * (size_t)c->seqlen);
    if (!z) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(dynamic, 16)
    for (int64_t i = 0; i < n_rows; ++i) {
      if (!z) continue;
      int b, h;
      int64_t pos;
      if (rows) {
        b = (int)rows[3 * i];
        h = (int)rows[3 * i + 1];
        pos = rows[3 * i + 2];
      } else {
        h = (int)(i % Hq);
        pos = (i / Hq) % c->seqlen;
        b = (int)(i / ((int64_t)Hq * c->seqlen));
      }
      int t = (int)(pos / tile_rows(c));
      int64_t bht = ((int64_t)b * units(c) + h / heads_per_unit(c)) * n + t;
      double l;
      attend_row(c, Q, K, V, kv_idx + bht * W, kv_cnt[bht], (double)softmax_scale, b, pos, h,
                 O + i * d, &l, z);
      if (lse) lse[i] = l;
    }
    free(z);
  }
  return fail ? -1 : 0;
}

/* ------------------------------------------------------- vertical-slash index lists */

/* VSPrefill page, Metodologia B.3: the sparse attention of query tile t reads the union of the
 * selected vertical columns and the selected slash diagonals.  At block granularity (this
 * build's reading): vertical entries are key-block indices, slash entries are block offsets
 * delta, tile t reads block t - delta, and the diagonal block t is always read (as in every
 * other list).  vert [B, Hq, NV] and slash [B, Hq, NS] end at their first negative entry;
 * entries beyond the tile (a vertical block > t, an offset > t) are skipped.  Output: the
 * union in ascending order, -1 padded to W entries, and its size. */
int oracle_vs_lists(const oc_cfg* c, const int32_t* vert, int NV, const int32_t* slash, int NS,
                    int32_t* kv_idx, int32_t* kv_cnt, int W) {
  const int n = c->seqlen / c->block, Hq = c->n_q_heads;
  int fail = 0;
#pragma omp parallel
  {
    unsigned char* in = (unsigned char*)malloc((size_t)n);
    if (!in) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for collapse(2) schedule(static)
    for (int bh = 0; bh < c->batch * Hq; ++bh)
      for (int t = 0; t < n; ++t) {
        if (!in) continue;
        memset(in, 0, (size_t)(t + 1));
        in[t] = 1;
        for (int e = 0; e < NV; ++e) {
          const int v = vert[(int64_t)bh * NV + e];
          if (v < 0) break;
          if (v <= t) in[v] = 1;
        }
        for (int e = 0; e < NS; ++e) {
          const int dlt = slash[(int64_t)bh * NS + e];
          if (dlt < 0) break;
          if (dlt <= t) in[t - dlt] = 1;
        }
        int32_t* out = kv_idx + ((int64_t)bh * n + t) * W;
        int m = 0;
        for (int j = 0; j <= t; ++j)
          if (in[j]) {
            if (m < W) out[m] = j;
            ++m;
          }
        if (m > W) {
#pragma omp atomic write
          fail = 2;
        }
        for (int e = m; e < W; ++e) out[e] = -1;
        kv_cnt[(int64_t)bh * n + t] = m < W ? m : W;
      }
    free(in);
  }
  return fail ? -fail : 0;
}

/* ------------------------------------------- decode with run-time termination (ART) */

/* ART page, sections 2.1-2.4: a decode query attends to the K/V cache block by block with an
 * online softmax; after each block the partial output's probe vector is compared with the
 * previous one, and the traversal stops once both the change of its L2 norm (below tau) and
 * its change of direction, 1 - cosine similarity (below phi), have held for `patience`
 * consecutive blocks.  Block 0 (the attention sink) is always evaluated first; the other
 * blocks follow recency-first (n-1, n-2, ..., 1), an order the online softmax is invariant to.
 * This build's readings: the probe is the partial output's first `probe` coordinates; the
 * stability of step k >= 1 compares steps k and k-1; stopping after step k (k >= patience)
 * keeps O^(k), the normalised output over the first k + 1 blocks of the order; patience 0
 * never stops.
 *
 * Q [B, Hq, d] (the decode tokens), K, V [B, N, Hkv, d]; the query attends to keys 0 .. N-1.
 * Everything in fp64.  Outputs per (b, h): dscale[k], ddir[k] for k = 0 .. n-1 (step 0 has
 * no predecessor: 0 and 0), the partial outputs O^(k) [n][d] when Opart is not NULL, and
 * stop = the number of blocks the rule processes (n when it never stops). */
int oracle_decode_art(const oc_cfg* c, const void* Q, const void* K, const void* V,
                      double softmax_scale, int probe, double tau, double phi, int patience,
                      double* dscale, double* ddir, double* Opart, int32_t* stop) {
  const int N = c->seqlen, blk = c->block, n = N / blk, d = c->head_dim;
  const int Hq = c->n_q_heads, Hkv = c->n_kv_heads, G = Hq / Hkv;
  if (probe < 1 || probe > d) return -2;
  int fail = 0;
#pragma omp parallel
  {
    double* acc = (double*)malloc(sizeof(double) * (size_t)d);
    double* prev = (double*)malloc(sizeof(double) * (size_t)probe);
    double* s = (double*)malloc(sizeof(double) * (size_t)blk);
    if (!acc || !prev || !s) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int bh = 0; bh < c->batch * Hq; ++bh) {
      if (!acc || !prev || !s) continue;
      const int b = bh / Hq, h = bh % Hq, g = h / G;
      double m = -INFINITY, l = 0.0;
      for (int ch = 0; ch < d; ++ch) acc[ch] = 0.0;
      for (int i = 0; i < probe; ++i) prev[i] = 0.0;
      int run = 0, stopped = n;
      for (int k = 0; k < n; ++k) {
        const int j = k == 0 ? 0 : n - k; /* block 0, then n-1, n-2, ..., 1 */
        double bm = -INFINITY;
        for (int r = 0; r < blk; ++r) {
          const int64_t pos = (int64_t)j * blk + r;
          double dot = 0.0;
          for (int ch = 0; ch < d; ++ch)
            dot += (double)elem(Q, c->in_dtype, ((int64_t)b * Hq + h) * d + ch) *
                   (double)elem(K, c->in_dtype, bshd(c, b, pos, g, Hkv, ch));
          s[r] = dot * softmax_scale;
          if (s[r] > bm) bm = s[r];
        }
        const double mn = bm > m ? bm : m;
        const double a = exp(m - mn);
        l *= a;
        for (int ch = 0; ch < d; ++ch) acc[ch] *= a;
        for (int r = 0; r < blk; ++r) {
          const double w = exp(s[r] - mn);
          l += w;
          const int64_t pos = (int64_t)j * blk + r;
          for (int ch = 0; ch < d; ++ch)
            acc[ch] += w * (double)elem(V, c->in_dtype, bshd(c, b, pos, g, Hkv, ch));
        }
        m = mn;
        double nx = 0.0, np = 0.0, dp = 0.0;
        for (int i = 0; i < probe; ++i) {
          const double x = acc[i] / l;
          nx += x * x;
          np += prev[i] * prev[i];
          dp += x * prev[i];
        }
        nx = sqrt(nx);
        np = sqrt(np);
        double dsc = 0.0, ddr = 0.0;
        if (k > 0) {
          dsc = fabs(nx - np);
          ddr = (nx > 0.0 && np > 0.0) ? 1.0 - dp / (nx * np) : 1.0;
        }
        dscale[(int64_t)bh * n + k] = dsc;
        ddir[(int64_t)bh * n + k] = ddr;
        for (int i = 0; i < probe; ++i) prev[i] = acc[i] / l;
        if (Opart)
          for (int ch = 0; ch < d; ++ch) Opart[((int64_t)bh * n + k) * d + ch] = acc[ch] / l;
        if (k > 0 && stopped == n && patience > 0) {
          run = (dsc < tau && ddr < phi) ? run + 1 : 0;
          if (run >= patience) stopped = k + 1;
        }
      }
      stop[bh] = stopped;
    }
    free(acc);
    free(prev);
    free(s);
  }
  return fail ? -1 : 0;
}

/* Per-layer threshold for a fixed gate from calibration runs (gated-selection page,
 * Metodologia step 4: the gate threshold is an empirical quantile per layer).  This build's
 * reading: the mean of the per-sequence quantile thresholds tau[0 .. B) over the sequences
 * where a tile can trip (finite tau), as an fp32 sum in index order divided by their count;
 * -inf when there is none. */
float oracle_calibrated_tau(const float* tau, int B) {
  float acc = 0.0f;
  int c = 0;
  for (int b = 0; b < B; ++b)
    if (isfinite(tau[b])) {
      acc = acc + tau[b];
      ++c;
    }
  return c > 0 ? acc / (float)c : -INFINITY;
}

/* Budget for tile t, exported so the tests can pin the schedule on its own. */
int oracle_budget(const oc_cfg* c, int t) { return budget(c, t); }

/* The library is built with FMA instructions enabled; report whether this CPU has them. */
int oracle_cpu_ok(void) {
  __builtin_cpu_init();
  return __builtin_cpu_supports("fma") ? 1 : 0;
}

/* Threads the oracle's parallel loops use (OpenMP's current maximum). */
#include <omp.h>
int oracle_threads(void) { return omp_get_max_threads(); }
