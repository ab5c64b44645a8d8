/*
 * mla_oracle.c -- plain, slow, float64 CPU oracle for Multi-head Latent
 * Attention (MLA) over a compressed latent KV cache, computed both ways.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header or constant with the
 * HIP library.
 *
 * What it computes (pages: "One guard, 110x off the verify step", section
 * "The defect"; mlx-lm PR #1817 "fix: Speed up multi-token decode by computing
 * the absorbed MLA threshold", opening paragraphs):  MLA caches, per token t, a
 * latent c_kv[t] (rank r) and a rope key k_pe[t] shared by every head.  The
 * attention of a block of L new query rows can be taken two mathematically
 * equivalent ways:
 *   absorbed      -- fold the key up-projection W_UK into the query, attend
 *                    against the latent itself, accumulate in latent space,
 *                    then up-project through W_UV;
 *   materialised  -- expand the cached latent into full per-head K and V,
 *                    then run ordinary attention.
 * Readings the pages leave open (all stated here, the same ones are used by
 * the tests):
 *   - W_UK is [H, n, r] and W_UV is [H, r, v]; the output is the per-head
 *     attention output before any output projection.
 *   - q_pe and k_pe arrive already rotated; k_pe is shared by all heads.
 *   - causal rule of a verify block: the L new rows are the last L positions
 *     of a sequence of Kv cached positions, so row i sees the first
 *     Kv - L + i + 1 positions.
 *   - scale is an input (the tests use 1/sqrt(n + rope)).
 *
 * Everything is float64, plain loops, no blocking, no fusion.  OpenMP only
 * parallelises the outermost independent loop (rows, or (sequence, head)).
 *
 * Layouts (row-major, contiguous):
 *   q_nope [B, L, H, n]   q_pe [B, L, H, rope]   q_lat [B, L, H, r]
 *   c_kv   [sumKv, r]     k_pe [sumKv, rope]     (sequence b owns positions
 *                                                 offsets[b] .. offsets[b+1]-1)
 *   w_uk   [H, n, r]      w_uv [H, r, v]
 *   K      [T, H, n+rope] V    [T, H, v]          out  [rows, v]
 * A "row id" is (b*L + i)*H + h.  Functions taking (nsel, sel) compute only
 * the listed row ids, writing out[k*v ...] for sel[k]; sel == NULL means all
 * B*L*H rows in order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Number of positions row i of a block of L rows may attend to, out of Kv. */
static int64_t visible(int64_t Kv, int64_t L, int64_t i) { return Kv - L + i + 1; }

/* Fold for one (row, head): ql[c] = sum_j q_nope[j] * W_UK[h, j, c]
 * ("One guard..." section "The defect": fold the up-projection into the query). */
static void fold_one(int64_t n, int64_t r, const double* qn, const double* wuk_h, double* ql) {
  for (int64_t c = 0; c < r; ++c) {
    double acc = 0.0;
    for (int64_t j = 0; j < n; ++j) acc += qn[j] * wuk_h[j * r + c];
    ql[c] = acc;
  }
}

/* Latent attention for one (row, head), given the folded query ql:
 *   s_t  = scale * (ql . c_kv[t] + q_pe . k_pe[t])      for t < vis
 *   w_t  = exp(s_t - max s),  Z = sum w_t
 *   ol   = sum_t w_t c_kv[t] / Z                        (latent space)
 *   out  = ol . W_UV[h]                                  (up-projection)
 */
static void latent_attend_one(int64_t r, int64_t v, int64_t rope, int64_t vis,
                              const double* ql, const double* qpe,
                              const double* ckv, const double* kpe,  /* first key of the sequence */
                              const double* wuv_h, double scale, double* out, double* s, double* ol) {
  double m = -INFINITY;
  for (int64_t t = 0; t < vis; ++t) {
    double acc = 0.0;
    for (int64_t c = 0; c < r; ++c) acc += ql[c] * ckv[t * r + c];
    for (int64_t p = 0; p < rope; ++p) acc += qpe[p] * kpe[t * rope + p];
    s[t] = scale * acc;
    if (s[t] > m) m = s[t];
  }
  double Z = 0.0;
  for (int64_t t = 0; t < vis; ++t) { s[t] = exp(s[t] - m); Z += s[t]; }
  for (int64_t c = 0; c < r; ++c) {
    double acc = 0.0;
    for (int64_t t = 0; t < vis; ++t) acc += s[t] * ckv[t * r + c];
    ol[c] = acc / Z;
  }
  for (int64_t k = 0; k < v; ++k) {
    double acc = 0.0;
    for (int64_t c = 0; c < r; ++c) acc += ol[c] * wuv_h[c * v + k];
    out[k] = acc;
  }
}

static int64_t max_kv(int64_t B, const int64_t* offsets) {
  int64_t m = 0;
  for (int64_t b = 0; b < B; ++b) if (offsets[b + 1] - offsets[b] > m) m = offsets[b + 1] - offsets[b];
  return m;
}

/* q_lat[row, h, :] = q_nope[row, h, :] . W_UK[h]   for rows = B*L. */
void oracle_fold(int64_t rows, int64_t H, int64_t n, int64_t r,
                 const double* q_nope, const double* w_uk, double* q_lat, int nthreads) {
  set_threads(nthreads);
  #pragma omp parallel for schedule(dynamic, 1)
  for (int64_t rh = 0; rh < rows * H; ++rh) {
    int64_t h = rh % H;
    fold_one(n, r, q_nope + rh * n, w_uk + h * n * r, q_lat + rh * r);
  }
}

/* Absorbed path starting from a given folded query q_lat (the attention half
 * of the absorbed path, i.e. what follows the fold). */
void oracle_latent_attention(int64_t r, int64_t v, int64_t rope, int64_t H, int64_t B, int64_t L,
                             const int64_t* offsets, const double* q_lat, const double* q_pe,
                             const double* c_kv, const double* k_pe, const double* w_uv,
                             double scale, int64_t nsel, const int64_t* sel, double* out, int nthreads) {
  set_threads(nthreads);
  int64_t total = sel ? nsel : B * L * H;
  int64_t kvmax = max_kv(B, offsets);
  #pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(kvmax > 0 ? kvmax : 1));
    double* ol = (double*)malloc(sizeof(double) * (size_t)r);
    #pragma omp for schedule(dynamic, 1)
    for (int64_t k = 0; k < total; ++k) {
      int64_t row = sel ? sel[k] : k;
      int64_t h = row % H, i = (row / H) % L, b = row / (H * L);
      int64_t off = offsets[b], Kv = offsets[b + 1] - offsets[b];
      latent_attend_one(r, v, rope, visible(Kv, L, i), q_lat + row * r, q_pe + row * rope,
                        c_kv + off * r, k_pe + off * rope, w_uv + h * r * v, scale, out + k * v, s, ol);
    }
    free(s); free(ol);
  }
}

/* Whole absorbed path: fold, then latent attention, then up-projection. */
void oracle_absorbed(int64_t r, int64_t n, int64_t v, int64_t rope, int64_t H, int64_t B, int64_t L,
                     const int64_t* offsets, const double* q_nope, const double* q_pe,
                     const double* c_kv, const double* k_pe, const double* w_uk, const double* w_uv,
                     double scale, int64_t nsel, const int64_t* sel, double* out, int nthreads) {
  set_threads(nthreads);
  int64_t total = sel ? nsel : B * L * H;
  int64_t kvmax = max_kv(B, offsets);
  #pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(kvmax > 0 ? kvmax : 1));
    double* ol = (double*)malloc(sizeof(double) * (size_t)r);
    double* ql = (double*)malloc(sizeof(double) * (size_t)r);
    #pragma omp for schedule(dynamic, 1)
    for (int64_t k = 0; k < total; ++k) {
      int64_t row = sel ? sel[k] : k;
      int64_t h = row % H, i = (row / H) % L, b = row / (H * L);
      int64_t off = offsets[b], Kv = offsets[b + 1] - offsets[b];
      fold_one(n, r, q_nope + row * n, w_uk + h * n * r, ql);
      latent_attend_one(r, v, rope, visible(Kv, L, i), ql, q_pe + row * rope,
                        c_kv + off * r, k_pe + off * rope, w_uv + h * r * v, scale, out + k * v, s, ol);
    }
    free(s); free(ol); free(ql);
  }
}

/* Expansion of the cache into full per-head keys and values
 * ("One guard..." section "The defect": expand the cached latent back into
 * full K and V).  For each listed position t (all T when tsel == NULL):
 *   K[t, h, j]     = sum_c W_UK[h, j, c] c_kv[t, c]      j < n
 *   K[t, h, n + p] = k_pe[t, p]                           (shared rope key)
 *   V[t, h, k]     = sum_c c_kv[t, c] W_UV[h, c, k]
 * With tsel, K and V hold only the listed positions, in list order. */
void oracle_expand(int64_t T, int64_t H, int64_t r, int64_t n, int64_t v, int64_t rope,
                   const double* c_kv, const double* k_pe, const double* w_uk, const double* w_uv,
                   int64_t ntsel, const int64_t* tsel, double* K, double* V, int nthreads) {
  set_threads(nthreads);
  int64_t total = tsel ? ntsel : T;
  int64_t dk = n + rope;
  #pragma omp parallel for schedule(dynamic, 1)
  for (int64_t k = 0; k < total; ++k) {
    int64_t t = tsel ? tsel[k] : k;
    for (int64_t h = 0; h < H; ++h) {
      for (int64_t j = 0; j < n; ++j) {
        double acc = 0.0;
        for (int64_t c = 0; c < r; ++c) acc += w_uk[(h * n + j) * r + c] * c_kv[t * r + c];
        K[(k * H + h) * dk + j] = acc;
      }
      for (int64_t p = 0; p < rope; ++p) K[(k * H + h) * dk + n + p] = k_pe[t * rope + p];
      for (int64_t kk = 0; kk < v; ++kk) {
        double acc = 0.0;
        for (int64_t c = 0; c < r; ++c) acc += c_kv[t * r + c] * w_uv[(h * r + c) * v + kk];
        V[(k * H + h) * v + kk] = acc;
      }
    }
  }
}

/* Ordinary causal attention over given per-head K and V (the attention half
 * of the materialised path).  The query is q_nope || q_pe:
 *   s_t = scale * (sum_j q_nope[j] K[t,h,j] + sum_p q_pe[p] K[t,h,n+p]),  t < vis
 *   out = sum_t exp(s_t - max) V[t,h,:] / sum_t exp(s_t - max)           */
void oracle_attention(int64_t n, int64_t v, int64_t rope, int64_t H, int64_t B, int64_t L,
                      const int64_t* offsets, const double* q_nope, const double* q_pe,
                      const double* K, const double* V, double scale,
                      int64_t nsel, const int64_t* sel, double* out, int nthreads) {
  set_threads(nthreads);
  int64_t total = sel ? nsel : B * L * H;
  int64_t kvmax = max_kv(B, offsets);
  int64_t dk = n + rope;
  #pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(kvmax > 0 ? kvmax : 1));
    #pragma omp for schedule(dynamic, 1)
    for (int64_t k = 0; k < total; ++k) {
      int64_t row = sel ? sel[k] : k;
      int64_t h = row % H, i = (row / H) % L, b = row / (H * L);
      int64_t off = offsets[b], Kv = offsets[b + 1] - offsets[b];
      int64_t vis = visible(Kv, L, i);
      const double* qn = q_nope + row * n;
      const double* qp = q_pe + row * rope;
      double m = -INFINITY;
      for (int64_t t = 0; t < vis; ++t) {
        const double* kr = K + ((off + t) * H + h) * dk;
        double acc = 0.0;
        for (int64_t j = 0; j < n; ++j) acc += qn[j] * kr[j];
        for (int64_t p = 0; p < rope; ++p) acc += qp[p] * kr[n + p];
        s[t] = scale * acc;
        if (s[t] > m) m = s[t];
      }
      double Z = 0.0;
      for (int64_t t = 0; t < vis; ++t) { s[t] = exp(s[t] - m); Z += s[t]; }
      for (int64_t kk = 0; kk < v; ++kk) {
        double acc = 0.0;
        for (int64_t t = 0; t < vis; ++t) acc += s[t] * V[((off + t) * H + h) * v + kk];
        out[k * v + kk] = acc / Z;
      }
    }
    free(s);
  }
}

/* Whole materialised path: for each (sequence, head) expand that head's K and
 * V over the sequence's positions, then attend with the same mask and scale.
 * One head at a time keeps memory small; the values are those of
 * oracle_expand followed by oracle_attention. */
void oracle_materialized(int64_t r, int64_t n, int64_t v, int64_t rope, int64_t H, int64_t B, int64_t L,
                         const int64_t* offsets, const double* q_nope, const double* q_pe,
                         const double* c_kv, const double* k_pe, const double* w_uk, const double* w_uv,
                         double scale, double* out /* [B*L*H, v] */, int nthreads) {
  set_threads(nthreads);
  int64_t kvmax = max_kv(B, offsets);
  #pragma omp parallel
  {
    double* Kn = (double*)malloc(sizeof(double) * (size_t)(kvmax > 0 ? kvmax : 1) * (size_t)(n > 0 ? n : 1));
    double* Vh = (double*)malloc(sizeof(double) * (size_t)(kvmax > 0 ? kvmax : 1) * (size_t)v);
    double* s = (double*)malloc(sizeof(double) * (size_t)(kvmax > 0 ? kvmax : 1));
    #pragma omp for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < B * H; ++bh) {
      int64_t b = bh / H, h = bh % H;
      int64_t off = offsets[b], Kv = offsets[b + 1] - offsets[b];
      for (int64_t t = 0; t < Kv; ++t) {
        const double* ck = c_kv + (off + t) * r;
        for (int64_t j = 0; j < n; ++j) {
          double acc = 0.0;
          for (int64_t c = 0; c < r; ++c) acc += w_uk[(h * n + j) * r + c] * ck[c];
          Kn[t * n + j] = acc;
        }
        for (int64_t kk = 0; kk < v; ++kk) {
          double acc = 0.0;
          for (int64_t c = 0; c < r; ++c) acc += ck[c] * w_uv[(h * r + c) * v + kk];
          Vh[t * v + kk] = acc;
        }
      }
      for (int64_t i = 0; i < L; ++i) {
        int64_t row = (b * L + i) * H + h;
        int64_t vis = visible(Kv, L, i);
        const double* qn = q_nope + row * n;
        const double* qp = q_pe + row * rope;
        double m = -INFINITY;
        for (int64_t t = 0; t < vis; ++t) {
          double acc = 0.0;
          for (int64_t j = 0; j < n; ++j) acc += qn[j] * Kn[t * n + j];
          for (int64_t p = 0; p < rope; ++p) acc += qp[p] * k_pe[(off + t) * rope + p];
          s[t] = scale * acc;
          if (s[t] > m) m = s[t];
        }
        double Z = 0.0;
        for (int64_t t = 0; t < vis; ++t) { s[t] = exp(s[t] - m); Z += s[t]; }
        for (int64_t kk = 0; kk < v; ++kk) {
          double acc = 0.0;
          for (int64_t t = 0; t < vis; ++t) acc += s[t] * Vh[t * v + kk];
          out[row * v + kk] = acc / Z;
        }
      }
    }
    free(Kn); free(Vh); free(s);
  }
}
