/* drive_oracle.c -- runs the float64 oracle (oracle/mla_oracle.c) on small
 * random problems, both routes, under -fsanitize=address,undefined; checks
 * that the routes agree (associativity of the two MLA forms) so that every
 * buffer is written and read.  A sanitizer report or a disagreement ends the
 * program with a non-zero status. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_fold(int64_t rows, int64_t H, int64_t n, int64_t r, const double* q_nope, const double* w_uk,
                 double* q_lat, int nthreads);
void oracle_latent_attention(int64_t r, int64_t v, int64_t rope, int64_t H, int64_t B, int64_t L,
                             const int64_t* offsets, const double* q_lat, const double* q_pe, const double* c_kv,
                             const double* k_pe, const double* w_uv, double scale, int64_t nsel, const int64_t* sel,
                             double* out, int nthreads);
void oracle_absorbed(int64_t r, int64_t n, int64_t v, int64_t rope, int64_t H, int64_t B, int64_t L,
                     const int64_t* offsets, const double* q_nope, const double* q_pe, const double* c_kv,
                     const double* k_pe, const double* w_uk, const double* w_uv, double scale, int64_t nsel,
                     const int64_t* sel, double* out, int nthreads);
void oracle_expand(int64_t T, int64_t H, int64_t r, int64_t n, int64_t v, int64_t rope, const double* c_kv,
                   const double* k_pe, const double* w_uk, const double* w_uv, int64_t ntsel, const int64_t* tsel,
                   double* K, double* V, int nthreads);
void oracle_attention(int64_t n, int64_t v, int64_t rope, int64_t H, int64_t B, int64_t L, const int64_t* offsets,
                      const double* q_nope, const double* q_pe, const double* K, const double* V, double scale,
                      int64_t nsel, const int64_t* sel, double* out, int nthreads);
void oracle_materialized(int64_t r, int64_t n, int64_t v, int64_t rope, int64_t H, int64_t B, int64_t L,
                         const int64_t* offsets, const double* q_nope, const double* q_pe, const double* c_kv,
                         const double* k_pe, const double* w_uk, const double* w_uv, double scale, double* out,
                         int nthreads);

static uint64_t state = 88172645463325252ull;
static double rnd(void) {   /* xorshift64, uniform in [-1, 1) */
  state ^= state << 13; state ^= state >> 7; state ^= state << 17;
  return (double)(state >> 11) / 4503599627370496.0 - 1.0;
}
static double* fill(size_t n) {
  double* p = (double*)malloc(sizeof(double) * (n ? n : 1));
  for (size_t i = 0; i < n; ++i) p[i] = rnd();
  return p;
}

int main(void) {
  int bad = 0;
  for (int it = 0; it < 40; ++it) {
    const int64_t r = 8 + 8 * (it % 4), n = 4 + (it % 3) * 4, v = 4 + (it % 5) * 2, rope = (it % 2) * 6;
    const int64_t H = 1 + it % 3, B = 1 + it % 4, L = 1 + it % 5;
    int64_t off[5] = {0};
    for (int64_t b = 0; b < B; ++b) off[b + 1] = off[b] + L + (it * 7 + b * 3) % 29;
    const int64_t T = off[B], rows = B * L * H;
    double *qn = fill((size_t)(B * L * H * n)), *qp = fill((size_t)(B * L * H * rope));
    double *ck = fill((size_t)(T * r)), *kp = fill((size_t)(T * rope));
    double *wk = fill((size_t)(H * n * r)), *wv = fill((size_t)(H * r * v));
    double *ql = fill((size_t)(B * L * H * r)), *K = fill((size_t)(T * H * (n + rope))), *V = fill((size_t)(T * H * v));
    double *o1 = fill((size_t)(rows * v)), *o2 = fill((size_t)(rows * v)), *o3 = fill((size_t)(rows * v));
    double *o4 = fill((size_t)(rows * v));
    const double scale = 1.0 / sqrt((double)(n + rope));
    oracle_absorbed(r, n, v, rope, H, B, L, off, qn, qp, ck, kp, wk, wv, scale, 0, NULL, o1, 1);
    oracle_materialized(r, n, v, rope, H, B, L, off, qn, qp, ck, kp, wk, wv, scale, o2, 1);
    oracle_fold(B * L, H, n, r, qn, wk, ql, 1);
    oracle_latent_attention(r, v, rope, H, B, L, off, ql, qp, ck, kp, wv, scale, 0, NULL, o3, 1);
    oracle_expand(T, H, r, n, v, rope, ck, kp, wk, wv, 0, NULL, K, V, 1);
    oracle_attention(n, v, rope, H, B, L, off, qn, qp, K, V, scale, 0, NULL, o4, 1);
    const int64_t sel[2] = {rows - 1, 0};
    double o5[2 * 16];
    oracle_absorbed(r, n, v, rope, H, B, L, off, qn, qp, ck, kp, wk, wv, scale, 2, sel, o5, 1);
    for (int64_t k = 0; k < rows * v; ++k) {
      const double e = fabs(o1[k] - o2[k]) + fabs(o1[k] - o3[k]) + fabs(o1[k] - o4[k]);
      if (!(e <= 1e-12)) ++bad;
    }
    for (int64_t k = 0; k < v; ++k)
      if (o5[k] != o1[(rows - 1) * v + k] || o5[v + k] != o1[k]) ++bad;
    free(qn); free(qp); free(ck); free(kp); free(wk); free(wv); free(ql); free(K); free(V);
    free(o1); free(o2); free(o3); free(o4);
  }
  printf("oracle driver: %d disagreements\n", bad);
  return bad == 0 ? 0 : 1;
}
