// bench_driver.cpp -- native timing loop for bench.py (built as a separate
// libmla_bench.so; not part of libmla's ABI).  Issues the absorbed verify
// step -- mla_fold_query, then mla_absorbed_attention (split pass and merge);
// over the fp8 cache mla_fold_query_fp8, then mla_absorbed_attention_fp8q --
// from C so that host launch cost stays below the GPU time per step, and times
// it with HIP events on the caller's stream.  The split pass and the merge are
// also timed alone, through their separate entry points.  Input sets are rotated so that a set is
// evicted from the caches before it is used again when enough sets are given.

#include "../../include/mla.h"

#include <hip/hip_runtime.h>

#include <vector>

namespace {

struct Sets {
  void* const* q_nope; void* const* q_pe; void* const* c_kv; void* const* k_pe;
  void* const* w_uk; void* const* w_uv; void* const* q_lat; float* const* out;
  void* const* codes; float* const* scales;   // fp8 cache (null: the bf16 cache)
  void* const* q8;                            // fp8 cache: the fold's E4M3 query blocks
};

int fold(const mla_geom* g, int B, int L, const Sets& s, int k, hipStream_t st) {
  if (s.codes) return mla_fold_query_fp8(g, B, L, s.q_nope[k], s.w_uk[k], s.q_pe[k], nullptr, s.q8[k], st);
  return mla_fold_query(g, MLA_BF16, (int64_t)B * L, s.q_nope[k], s.w_uk[k], s.q_lat[k], st);
}

int splits(const mla_geom* g, int B, int L, const Sets& s, int k, const int32_t* off_h, const int32_t* off_d,
           float scale, void* ws, size_t ws_bytes, hipStream_t st) {
  if (s.codes)
    return mla_absorbed_splits_fp8q(g, B, L, s.q8[k], s.codes[k], s.scales[k], off_h, off_d, scale, ws, ws_bytes, st);
  return mla_absorbed_splits(g, MLA_BF16, B, L, s.q_lat[k], s.q_pe[k], s.c_kv[k], s.k_pe[k], off_h, off_d, scale,
                             ws, ws_bytes, st);
}

int attention(const mla_geom* g, int B, int L, const Sets& s, int k, const int32_t* off_h, const int32_t* off_d,
              float scale, void* ws, size_t ws_bytes, hipStream_t st) {
  if (s.codes)
    return mla_absorbed_attention_fp8q(g, B, L, s.q8[k], s.codes[k], s.scales[k], off_h, off_d, s.w_uv[k], scale,
                                       s.out[k], ws, ws_bytes, st);
  return mla_absorbed_attention(g, MLA_BF16, B, L, s.q_lat[k], s.q_pe[k], s.c_kv[k], s.k_pe[k], off_h, off_d,
                                s.w_uv[k], scale, s.out[k], ws, ws_bytes, st);
}

int step(const mla_geom* g, int B, int L, const Sets& s, int k, const int32_t* off_h, const int32_t* off_d,
         float scale, void* ws, size_t ws_bytes, hipStream_t st, hipEvent_t* ev) {
  int rc;
  if (ev) hipEventRecord(ev[0], st);
  if ((rc = fold(g, B, L, s, k, st))) return rc;
  if (ev) hipEventRecord(ev[1], st);
  if ((rc = attention(g, B, L, s, k, off_h, off_d, scale, ws, ws_bytes, st))) return rc;
  if (ev) hipEventRecord(ev[2], st);
  return 0;
}

}  // namespace

extern "C" {

// res[0] us/step, plain back-to-back steps (events only around the run)
// res[1] us fold, res[2] us attention call (split pass + merge) (per-call means,
//        evented run; each includes the dispatch gap before its first kernel)
// res[3] unused (0)
// res[4] us/step of the evented run
// res[5] us per mla_absorbed_splits launch, launches back to back over the same
//        rotation of input sets (events only around the run)
// res[6] us per mla_absorbed_merge launch, back to back (same rotation)
// res[7] us per mla_fold_query launch, back to back (same rotation)
// codes / scales: per input set, the fp8 cache (mla_quantize_latent_fp8) to use
// instead of c_kv / k_pe, or null; q8: then per set the query block buffer
// (mla_query_fp8_bytes) that mla_fold_query_fp8 fills
int mlab_absorbed_run(const mla_geom* g, int B, int L, int nsets, void* const* q_nope, void* const* q_pe,
                      void* const* c_kv, void* const* k_pe, void* const* w_uk, void* const* w_uv,
                      void* const* q_lat, float* const* out, const int32_t* off_h, const int32_t* off_d,
                      float scale, void* ws, size_t ws_bytes, void* stream, int warmup, int steps, double* res,
                      void* const* codes, float* const* scales, void* const* q8) {
  hipStream_t st = (hipStream_t)stream;
  if (codes && !q8) return MLA_E_NULL;
  Sets s{q_nope, q_pe, c_kv, k_pe, w_uk, w_uv, q_lat, out, codes, scales, q8};
  int rc;
  for (int i = 0; i < warmup; ++i)
    if ((rc = step(g, B, L, s, i % nsets, off_h, off_d, scale, ws, ws_bytes, st, nullptr))) return rc;
  hipEvent_t a, b;
  hipEventCreate(&a);
  hipEventCreate(&b);
  hipStreamSynchronize(st);
  hipEventRecord(a, st);
  for (int i = 0; i < steps; ++i)
    if ((rc = step(g, B, L, s, i % nsets, off_h, off_d, scale, ws, ws_bytes, st, nullptr))) return rc;
  hipEventRecord(b, st);
  hipStreamSynchronize(st);
  float ms = 0.f;
  hipEventElapsedTime(&ms, a, b);
  res[0] = 1e3 * ms / steps;

  std::vector<hipEvent_t> ev((size_t)steps * 3);
  for (auto& e : ev) hipEventCreate(&e);
  hipStreamSynchronize(st);
  for (int i = 0; i < steps; ++i)
    if ((rc = step(g, B, L, s, i % nsets, off_h, off_d, scale, ws, ws_bytes, st, &ev[(size_t)i * 3]))) return rc;
  hipStreamSynchronize(st);
  double t[2] = {0, 0};
  for (int i = 0; i < steps; ++i) {
    for (int j = 0; j < 2; ++j) {
      float x = 0.f;
      hipEventElapsedTime(&x, ev[(size_t)i * 3 + j], ev[(size_t)i * 3 + j + 1]);
      t[j] += x;
    }
  }
  float whole = 0.f;
  hipEventElapsedTime(&whole, ev[0], ev[(size_t)(steps - 1) * 3 + 2]);
  for (int j = 0; j < 2; ++j) res[1 + j] = 1e3 * t[j] / steps;
  res[3] = 0.0;
  res[4] = 1e3 * whole / steps;

  // split launches alone (q_lat or q8 of every set was written by the steps above)
  hipStreamSynchronize(st);
  hipEventRecord(a, st);
  for (int i = 0; i < steps; ++i) {
    const int k = i % nsets;
    if ((rc = splits(g, B, L, s, k, off_h, off_d, scale, ws, ws_bytes, st))) return rc;
  }
  hipEventRecord(b, st);
  hipStreamSynchronize(st);
  hipEventElapsedTime(&ms, a, b);
  res[5] = 1e3 * ms / steps;

  hipEventRecord(a, st);
  for (int i = 0; i < steps; ++i) {
    const int k = i % nsets;
    if ((rc = mla_absorbed_merge(g, MLA_BF16, B, L, off_h, off_d, s.w_uv[k], s.out[k], ws, ws_bytes, st))) return rc;
  }
  hipEventRecord(b, st);
  hipStreamSynchronize(st);
  hipEventElapsedTime(&ms, a, b);
  res[6] = 1e3 * ms / steps;

  hipEventRecord(a, st);
  for (int i = 0; i < steps; ++i) {
    const int k = i % nsets;
    if ((rc = fold(g, B, L, s, k, st))) return rc;
  }
  hipEventRecord(b, st);
  hipStreamSynchronize(st);
  hipEventElapsedTime(&ms, a, b);
  res[7] = 1e3 * ms / steps;
  for (auto& e : ev) hipEventDestroy(e);
  hipEventDestroy(a);
  hipEventDestroy(b);
  return hipGetLastError() == hipSuccess ? 0 : MLA_E_HIP;
}

}  // extern "C"
