// api.cpp -- the C ABI of libmla (declared in include/mla.h): argument
// validation on the host, split-KV planning, and kernel launches.  No call
// here allocates, frees, copies or synchronises.

#include "../../include/mla.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "internal.h"

using namespace mla;

namespace {

constexpr int kCUs = 256;            // MI355X compute units (planning target)
constexpr int kTile = 64;            // positions per attention tile, query rows per workgroup
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool dtype_ok(mla_dtype dt) { return dt == MLA_F32 || dt == MLA_BF16; }

int check_geom(const mla_geom* g) {
  if (!g) return MLA_E_NULL;
  if (g->r < 1 || g->n < 0 || g->v < 1 || g->rope < 0 || g->heads < 1) return MLA_E_SHAPE;
  return MLA_OK;
}

// Offsets: B >= 1, off[0] >= 0, every Kv_b >= L, and the packed length fits int32.
int check_offsets(int32_t B, int32_t L, const int32_t* off) {
  if (!off) return MLA_E_NULL;
  if (B < 1 || L < 1) return MLA_E_SHAPE;
  if (off[0] < 0) return MLA_E_SHAPE;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t kv = (int64_t)off[b + 1] - (int64_t)off[b];
    if (kv < L) return MLA_E_SHAPE;
  }
  return MLA_OK;
}

// Split-KV plan.  A workgroup of the bf16 kernels takes 64 query rows x one
// split; splits hold an even number of 64-position tiles (the kernel takes
// tiles in pairs, one per LDS buffer), at least two.
//   B == 1, bf16: the split count minimises a model of the kernel pair in
//     units of one tile's time: rounds of workgroups over the CUs x (tiles per
//     split + 2 for the prologue and epilogue), plus the merge's read-back of
//     the partial sums (8 MiB per unit).  Rounds matter: 398 workgroups on 256
//     CUs take two full rounds.
//   otherwise: about one workgroup per CU for one sequence, four per CU for a
//     batch (variable lengths need the slack to balance).
int make_plan(int32_t B, int32_t L, int32_t H, const int32_t* off, int rows_slot, int head_slots, int DV,
              int o_elem_bytes, bool bf16, SplitPlan* p) {
  const int64_t row_tiles = (rows_slot + kTile - 1) / kTile;
  int64_t total_tiles = 0;
  for (int32_t b = 0; b < B; ++b) total_tiles += (off[b + 1] - off[b] + kTile - 1) / kTile;
  const int64_t units = row_tiles * head_slots * total_tiles;
  const int64_t target = (int64_t)kCUs * (B > 1 ? 4 : 1);
  auto even = [](int64_t t) { return std::max<int64_t>(2, (t + 1) / 2 * 2); };
  int64_t chunk_tiles = even((units + target - 1) / target);
  if (B == 1 && bf16) {
    const int64_t wg_per_split = row_tiles * head_slots;
    const double merge_unit = (double)rows_slot * head_slots * DV * o_elem_bytes / (8.0 * 1024 * 1024);
    double best = -1.0;
    const int64_t smax = std::min<int64_t>(total_tiles, 8 * kCUs);
    for (int64_t s = 1; s <= smax; ++s) {
      const int64_t ct = even((total_tiles + s - 1) / s);
      const int64_t ns = (total_tiles + ct - 1) / ct;
      const int64_t rounds = (ns * wg_per_split + kCUs - 1) / kCUs;
      const double cost = (double)rounds * (double)(ct + 2) + merge_unit * (double)ns;
      if (best < 0.0 || cost < best) { best = cost; chunk_tiles = ct; }
    }
  }
  if (chunk_tiles * kTile > INT32_MAX) return MLA_E_SHAPE;
  const int chunk = (int)(chunk_tiles * kTile);
  int64_t splits = 0;
  for (int32_t b = 0; b < B; ++b) splits += (off[b + 1] - off[b] + chunk - 1) / chunk;
  const int64_t items = splits * head_slots * row_tiles;
  const int64_t f32_items = splits * head_slots * rows_slot;
  if (items > INT32_MAX || f32_items > INT32_MAX || splits > INT32_MAX) return MLA_E_SHAPE;
  p->chunk = chunk;
  p->n_splits = (int)splits;
  p->row_tiles = (int)row_tiles;
  p->head_slots = head_slots;
  p->n_items = (int)items;
  const size_t rows_total = (size_t)L * H;
  p->ws_o_bytes = (size_t)splits * rows_total * DV * o_elem_bytes;
  p->ws_ml_floats = (size_t)splits * rows_total * 2;
  p->ws_bytes = align_up(p->ws_o_bytes) + align_up(p->ws_ml_floats * 4);
  return MLA_OK;
}

int absorbed_supported(const mla_geom* g, mla_dtype dt) {
  if (dt == MLA_BF16) {
    if (g->r != 512 || !(g->rope == 0 || g->rope == 64) || g->v % 64 != 0)
      return MLA_E_UNSUPPORTED;
  } else {
    if (g->r > 1024 || g->r + g->rope > 1152 || g->v > 1024) return MLA_E_UNSUPPORTED;
  }
  return MLA_OK;
}

int materialized_supported(const mla_geom* g, mla_dtype dt) {
  if (dt == MLA_BF16) {
    if (!materialized_bf16_supported(g->n, g->rope, g->v)) return MLA_E_UNSUPPORTED;
  } else {
    if (g->n + g->rope > 1152 || g->v > 1024) return MLA_E_UNSUPPORTED;
  }
  return MLA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_E_HIP; }

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_E_NULL: return "null pointer";
    case MLA_E_SHAPE: return "size or offset out of range";
    case MLA_E_UNSUPPORTED: return "geometry or dtype not supported";
    case MLA_E_WORKSPACE: return "workspace missing or too small";
    case MLA_E_HIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

int mla_version(void) { return 1; }

int mla_select_path(const mla_geom* g, int64_t L, int64_t T, int32_t* path_out, int64_t* max_absorbed_out) {
  if (!g || !path_out) return MLA_E_NULL;
  if (g->r < 1 || g->n < 0 || g->v < 0 || L < 1 || T < 0 || (T > 0 && T < L)) return MLA_E_SHAPE;
  const __int128 r = g->r, d = (__int128)g->n + g->v;
  const __int128 denom = 2 * r - d;
  __int128 m;
  if (denom <= 0) {
    m = 1;
  } else if (T == 0) {
    m = (r * d) / denom;                       // floor: both operands positive
  } else {
    const __int128 t = T;
    m = (t * r * d) / (r * d + t * denom);     // absorbed while L <= T r d / (r d + T (2r - d))
  }
  if (m < 1) m = 1;
  if (m > (__int128)INT64_MAX) m = INT64_MAX;
  *path_out = ((__int128)L <= m) ? MLA_ABSORBED : MLA_MATERIALIZED;
  if (max_absorbed_out) *max_absorbed_out = (int64_t)m;
  return MLA_OK;
}

int mla_draft_cap(const double* verify_cost, int32_t n_widths, double p, double drafter, int32_t* cap_out,
                  double* speedup_out, double* speedup_by_cap) {
  if (!verify_cost || !cap_out || !speedup_out) return MLA_E_NULL;
  if (n_widths < 1 || !(p >= 0.0 && p <= 1.0) || !(drafter >= 0.0) || !std::isfinite(drafter)) return MLA_E_SHAPE;
  for (int32_t w = 0; w < n_widths; ++w)
    if (!(verify_cost[w] > 0.0) || !std::isfinite(verify_cost[w])) return MLA_E_SHAPE;
  int32_t cap = 0;
  double best = 1.0, acc = 1.0, term = 1.0;
  if (speedup_by_cap) speedup_by_cap[0] = 1.0;
  for (int32_t c = 1; c < n_widths; ++c) {
    term *= p;                 // p^c
    acc += term;               // tokens committed per round with cap c
    const double s = acc / (drafter + verify_cost[c] / verify_cost[0]);
    if (speedup_by_cap) speedup_by_cap[c] = s;
    if (s > best) {
      best = s;
      cap = c;
    }
  }
  *cap_out = cap;
  *speedup_out = best;
  return MLA_OK;
}

int mla_fold_query(const mla_geom* g, mla_dtype dt, int64_t rows, const void* q_nope, const void* w_uk,
                   void* q_lat, void* stream) {
  int st = check_geom(g);
  if (st) return st;
  if (!dtype_ok(dt)) return MLA_E_UNSUPPORTED;
  if (rows < 1 || g->n < 1 || rows * g->heads > INT32_MAX) return MLA_E_SHAPE;
  if (!q_nope || !w_uk || !q_lat) return MLA_E_NULL;
  if (dt == MLA_BF16 && (g->n % 32 != 0 || g->n > 512 || g->r % 64 != 0)) return MLA_E_UNSUPPORTED;
  return hip_status(fold_query(dt == MLA_BF16 ? kBF16 : kF32, (int)rows, g->heads, g->n, g->r, q_nope, w_uk,
                               q_lat, (hipStream_t)stream));
}

int mla_absorbed_workspace_size(const mla_geom* g, mla_dtype dt, int32_t B, int32_t L,
                                const int32_t* kv_offsets_host, size_t* bytes_out) {
  int st = check_geom(g);
  if (st) return st;
  if (!dtype_ok(dt)) return MLA_E_UNSUPPORTED;
  if (!bytes_out) return MLA_E_NULL;
  if ((st = check_offsets(B, L, kv_offsets_host))) return st;
  if ((int64_t)L * g->heads > INT32_MAX / 64) return MLA_E_SHAPE;
  if ((st = absorbed_supported(g, dt))) return st;
  SplitPlan p{};
  if ((st = make_plan(B, L, g->heads, kv_offsets_host, L * g->heads, 1, g->r, dt == MLA_BF16 ? 2 : 4, dt == MLA_BF16, &p)))
    return st;
  *bytes_out = p.ws_bytes;
  return MLA_OK;
}

namespace {

// Validation and planning shared by the absorbed launches.  need_inputs:
// the split pass reads q_lat, q_pe, c_kv, k_pe; need_merge: the merge reads
// w_uv and writes out.
int absorbed_prepare(const mla_geom* g, mla_dtype dt, int32_t B, int32_t L, const void* q_lat, const void* q_pe,
                     const void* c_kv, const void* k_pe, const int32_t* off_h, const int32_t* off_d,
                     const void* w_uv, const float* out, void* workspace, size_t workspace_bytes, float scale,
                     bool need_inputs, bool need_merge, AbsorbedLaunch* q) {
  int st = check_geom(g);
  if (st) return st;
  if (!dtype_ok(dt)) return MLA_E_UNSUPPORTED;
  if ((st = check_offsets(B, L, off_h))) return st;
  if ((int64_t)L * g->heads > INT32_MAX / 64) return MLA_E_SHAPE;
  if (!off_d) return MLA_E_NULL;
  if (need_inputs) {
    if (!q_lat || !c_kv) return MLA_E_NULL;
    if (g->rope > 0 && (!q_pe || !k_pe)) return MLA_E_NULL;
  }
  if (need_merge && (!w_uv || !out)) return MLA_E_NULL;
  if ((st = absorbed_supported(g, dt))) return st;
  SplitPlan p{};
  if ((st = make_plan(B, L, g->heads, off_h, L * g->heads, 1, g->r, dt == MLA_BF16 ? 2 : 4, dt == MLA_BF16, &p)))
    return st;
  if (!workspace || workspace_bytes < p.ws_bytes) return MLA_E_WORKSPACE;
  q->r = g->r; q->rope = g->rope; q->v_dim = g->v; q->H = g->heads; q->B = B; q->L = L;
  q->q_lat = q_lat; q->q_pe = q_pe; q->c_kv = c_kv; q->k_pe = k_pe; q->w_uv = w_uv;
  q->off_dev = off_d; q->scale = scale;
  q->off0 = off_h[0]; q->kv1 = off_h[1] - off_h[0];
  q->ws_o = workspace;
  q->ws_ml = (float*)((char*)workspace + align_up(p.ws_o_bytes));
  q->plan = p;
  return MLA_OK;
}

int absorbed_split_launch(const AbsorbedLaunch& q, mla_dtype dt, hipStream_t s) {
  return hip_status(dt == MLA_BF16 ? absorbed_attn_bf16(q, s) : attn_f32(&q, nullptr, s));
}

}  // namespace

int mla_absorbed_attention(const mla_geom* g, mla_dtype dt, int32_t B, int32_t L, const void* q_lat,
                           const void* q_pe, const void* c_kv, const void* k_pe, const int32_t* kv_offsets_host,
                           const int32_t* kv_offsets_dev, const void* w_uv, float scale, float* out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  AbsorbedLaunch q{};
  int st = absorbed_prepare(g, dt, B, L, q_lat, q_pe, c_kv, k_pe, kv_offsets_host, kv_offsets_dev, w_uv, out,
                            workspace, workspace_bytes, scale, true, true, &q);
  if (st) return st;
  hipStream_t s = (hipStream_t)stream;
  if ((st = absorbed_split_launch(q, dt, s))) return st;
  return hip_status(combine_upproj(q, dt == MLA_BF16 ? kBF16 : kF32, out, s));
}

int mla_absorbed_attention_noalloc(const mla_geom* g, mla_dtype dt, int32_t B, int32_t L, const void* q_lat,
                                   const void* q_pe, const void* c_kv, const void* k_pe,
                                   const int32_t* kv_offsets_host, const int32_t* kv_offsets_dev, const void* w_uv,
                                   float scale, float* out, void* stream) {
  // size check first: the planned partials must fit the static scratch array
  AbsorbedLaunch q{};
  void* scratch = nullptr;
  int st = absorbed_prepare(g, dt, B, L, q_lat, q_pe, c_kv, k_pe, kv_offsets_host, kv_offsets_dev, w_uv, out,
                            reinterpret_cast<void*>(kAlign), kScratchBytes, scale, true, true, &q);
  if (st) return st;
  if ((st = hip_status(scratch_address(&scratch)))) return st;
  q.ws_o = scratch;
  q.ws_ml = (float*)((char*)scratch + align_up(q.plan.ws_o_bytes));
  hipStream_t s = (hipStream_t)stream;
  if ((st = absorbed_split_launch(q, dt, s))) return st;
  return hip_status(combine_upproj(q, dt == MLA_BF16 ? kBF16 : kF32, out, s));
}

int mla_absorbed_splits(const mla_geom* g, mla_dtype dt, int32_t B, int32_t L, const void* q_lat,
                        const void* q_pe, const void* c_kv, const void* k_pe, const int32_t* kv_offsets_host,
                        const int32_t* kv_offsets_dev, float scale, void* workspace, size_t workspace_bytes,
                        void* stream) {
  AbsorbedLaunch q{};
  int st = absorbed_prepare(g, dt, B, L, q_lat, q_pe, c_kv, k_pe, kv_offsets_host, kv_offsets_dev, nullptr,
                            nullptr, workspace, workspace_bytes, scale, true, false, &q);
  if (st) return st;
  return absorbed_split_launch(q, dt, (hipStream_t)stream);
}

int mla_absorbed_merge(const mla_geom* g, mla_dtype dt, int32_t B, int32_t L, const int32_t* kv_offsets_host,
                       const int32_t* kv_offsets_dev, const void* w_uv, float* out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  AbsorbedLaunch q{};
  int st = absorbed_prepare(g, dt, B, L, nullptr, nullptr, nullptr, nullptr, kv_offsets_host, kv_offsets_dev,
                            w_uv, out, workspace, workspace_bytes, 0.f, false, true, &q);
  if (st) return st;
  return hip_status(combine_upproj(q, dt == MLA_BF16 ? kBF16 : kF32, out, (hipStream_t)stream));
}

int mla_quantize_latent_fp8(const mla_geom* g, int64_t T, const void* c_kv, const void* k_pe, void* codes,
                            float* scales, void* stream) {
  int st = check_geom(g);
  if (st) return st;
  if (T < 1 || T > INT32_MAX) return MLA_E_SHAPE;
  if (!c_kv || !codes || !scales) return MLA_E_NULL;
  if (g->rope > 0 && !k_pe) return MLA_E_NULL;
  if (g->r % 8 != 0 || g->rope % 8 != 0 || (g->r + g->rope) / 8 > 128) return MLA_E_UNSUPPORTED;
  return hip_status(quantize_latent_fp8(T, g->r, g->rope, c_kv, k_pe, codes, scales, (hipStream_t)stream));
}

namespace {
int absorbed_prepare_fp8(const mla_geom* g, int32_t B, int32_t L, const void* q_lat, const void* q_pe,
                         const void* codes, const float* scales, const int32_t* off_h, const int32_t* off_d,
                         const void* w_uv, const float* out, void* workspace, size_t workspace_bytes, float scale,
                         bool need_merge, AbsorbedLaunch* q) {
  if (!codes || !scales) return MLA_E_NULL;
  if (!g) return MLA_E_NULL;
  if (g->r != 512 || !(g->rope == 0 || g->rope == 64)) return MLA_E_UNSUPPORTED;
  return absorbed_prepare(g, MLA_BF16, B, L, q_lat, q_pe, codes, g->rope > 0 ? codes : nullptr, off_h, off_d, w_uv,
                          out, workspace, workspace_bytes, scale, true, need_merge, q);
}
}  // namespace

int mla_absorbed_splits_fp8(const mla_geom* g, int32_t B, int32_t L, const void* q_lat, const void* q_pe,
                            const void* codes, const float* scales, const int32_t* kv_offsets_host,
                            const int32_t* kv_offsets_dev, float scale, void* workspace, size_t workspace_bytes,
                            void* stream) {
  AbsorbedLaunch q{};
  int st = absorbed_prepare_fp8(g, B, L, q_lat, q_pe, codes, scales, kv_offsets_host, kv_offsets_dev, nullptr,
                                nullptr, workspace, workspace_bytes, scale, false, &q);
  if (st) return st;
  return hip_status(absorbed_attn_fp8(q, codes, scales, (hipStream_t)stream));
}

int mla_absorbed_attention_fp8(const mla_geom* g, int32_t B, int32_t L, const void* q_lat, const void* q_pe,
                               const void* codes, const float* scales, const int32_t* kv_offsets_host,
                               const int32_t* kv_offsets_dev, const void* w_uv, float scale, float* out,
                               void* workspace, size_t workspace_bytes, void* stream) {
  AbsorbedLaunch q{};
  int st = absorbed_prepare_fp8(g, B, L, q_lat, q_pe, codes, scales, kv_offsets_host, kv_offsets_dev, w_uv, out,
                                workspace, workspace_bytes, scale, true, &q);
  if (st) return st;
  hipStream_t s = (hipStream_t)stream;
  if ((st = hip_status(absorbed_attn_fp8(q, codes, scales, s)))) return st;
  return hip_status(combine_upproj(q, kBF16, out, s));
}

int mla_query_fp8_bytes(const mla_geom* g, int32_t B, int32_t L, size_t* bytes_out) {
  int st = check_geom(g);
  if (st) return st;
  if (!bytes_out) return MLA_E_NULL;
  if (B < 1 || L < 1 || (int64_t)L * g->heads > INT32_MAX / 64) return MLA_E_SHAPE;
  *bytes_out = (size_t)B * (size_t)(((int64_t)L * g->heads + 31) / 32) * kQ8TileBytes;
  return MLA_OK;
}

int mla_fold_query_fp8(const mla_geom* g, int32_t B, int32_t L, const void* q_nope, const void* w_uk,
                       const void* q_pe, void* q_lat, void* q8, void* stream) {
  int st = check_geom(g);
  if (st) return st;
  if (B < 1 || L < 1 || (int64_t)B * L * g->heads > INT32_MAX / 64) return MLA_E_SHAPE;
  if (!q_nope || !w_uk || !q8) return MLA_E_NULL;
  if (g->rope > 0 && !q_pe) return MLA_E_NULL;
  if (g->r != 512 || !(g->rope == 0 || g->rope == 64) || g->n % 32 != 0 || g->n > 512) return MLA_E_UNSUPPORTED;
  return hip_status(fold_query_fp8(B, L, g->heads, g->n, g->rope, q_nope, w_uk, q_pe, q_lat, q8, (hipStream_t)stream));
}

int mla_absorbed_splits_fp8q(const mla_geom* g, int32_t B, int32_t L, const void* q8, const void* codes,
                             const float* scales, const int32_t* kv_offsets_host, const int32_t* kv_offsets_dev,
                             float scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q8) return MLA_E_NULL;
  AbsorbedLaunch q{};
  int st = absorbed_prepare_fp8(g, B, L, q8, q8, codes, scales, kv_offsets_host, kv_offsets_dev, nullptr, nullptr,
                                workspace, workspace_bytes, scale, false, &q);
  if (st) return st;
  q.q8 = q8;
  return hip_status(absorbed_attn_fp8(q, codes, scales, (hipStream_t)stream));
}

int mla_absorbed_attention_fp8q(const mla_geom* g, int32_t B, int32_t L, const void* q8, const void* codes,
                                const float* scales, const int32_t* kv_offsets_host, const int32_t* kv_offsets_dev,
                                const void* w_uv, float scale, float* out, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (!q8) return MLA_E_NULL;
  AbsorbedLaunch q{};
  int st = absorbed_prepare_fp8(g, B, L, q8, q8, codes, scales, kv_offsets_host, kv_offsets_dev, w_uv, out,
                                workspace, workspace_bytes, scale, true, &q);
  if (st) return st;
  q.q8 = q8;
  hipStream_t s = (hipStream_t)stream;
  if ((st = hip_status(absorbed_attn_fp8(q, codes, scales, s)))) return st;
  return hip_status(combine_upproj(q, kBF16, out, s));
}

namespace {
// Selections: B >= 1, sel_off[0] >= 0, 1 <= k_b <= Kv_b for every sequence.
int check_selection(int32_t B, const int32_t* kv_off, const int32_t* sel_off) {
  if (!sel_off) return MLA_E_NULL;
  if (sel_off[0] < 0) return MLA_E_SHAPE;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t k = (int64_t)sel_off[b + 1] - sel_off[b];
    if (k < 1 || k > (int64_t)kv_off[b + 1] - kv_off[b]) return MLA_E_SHAPE;
  }
  return MLA_OK;
}
}  // namespace

int mla_absorbed_sparse_workspace_size(const mla_geom* g, int32_t B, int32_t L, const int32_t* kv_offsets_host,
                                       const int32_t* sel_offsets_host, size_t* bytes_out) {
  int st = check_geom(g);
  if (st) return st;
  if (!bytes_out) return MLA_E_NULL;
  if ((st = check_offsets(B, L, kv_offsets_host))) return st;
  if ((st = check_selection(B, kv_offsets_host, sel_offsets_host))) return st;
  if ((int64_t)L * g->heads > INT32_MAX / 64) return MLA_E_SHAPE;
  SplitPlan p{};
  if ((st = make_plan(B, L, g->heads, sel_offsets_host, L * g->heads, 1, g->r, 2, true, &p))) return st;
  *bytes_out = p.ws_bytes;
  return MLA_OK;
}

namespace {
// Validation and planning shared by the selected-position calls (bf16 cache:
// c_kv / k_pe; fp8 cache: codes / scales, passed as c_kv / k_pe = codes).
int sparse_prepare(const mla_geom* g, int32_t B, int32_t L, const void* q_lat, const void* q_pe, const void* c_kv,
                   const void* k_pe, const int32_t* kv_offsets_host, const int32_t* kv_offsets_dev, const int32_t* sel,
                   const int32_t* sel_offsets_host, const int32_t* sel_offsets_dev, const void* w_uv, float scale,
                   const float* out, void* workspace, size_t workspace_bytes, AbsorbedLaunch* q) {
  int st = check_geom(g);
  if (st) return st;
  if ((st = check_offsets(B, L, kv_offsets_host))) return st;
  if ((st = check_selection(B, kv_offsets_host, sel_offsets_host))) return st;
  if ((int64_t)L * g->heads > INT32_MAX / 64) return MLA_E_SHAPE;
  if (!kv_offsets_dev || !sel || !sel_offsets_dev || !q_lat || !c_kv || !w_uv || !out) return MLA_E_NULL;
  if (g->rope > 0 && (!q_pe || !k_pe)) return MLA_E_NULL;
  if ((st = absorbed_supported(g, MLA_BF16))) return st;
  SplitPlan p{};
  if ((st = make_plan(B, L, g->heads, sel_offsets_host, L * g->heads, 1, g->r, 2, true, &p))) return st;
  if (!workspace || workspace_bytes < p.ws_bytes) return MLA_E_WORKSPACE;
  q->r = g->r; q->rope = g->rope; q->v_dim = g->v; q->H = g->heads; q->B = B; q->L = L;
  q->q_lat = q_lat; q->q_pe = q_pe; q->c_kv = c_kv; q->k_pe = k_pe; q->w_uv = w_uv;
  q->off_dev = sel_offsets_dev; q->scale = scale;   // splits and merge run over the selections
  q->off0 = sel_offsets_host[0]; q->kv1 = sel_offsets_host[1] - sel_offsets_host[0];
  q->ws_o = workspace;
  q->ws_ml = (float*)((char*)workspace + align_up(p.ws_o_bytes));
  q->plan = p;
  return MLA_OK;
}
}  // namespace

int mla_absorbed_attention_sparse(const mla_geom* g, int32_t B, int32_t L, const void* q_lat, const void* q_pe,
                                  const void* c_kv, const void* k_pe, const int32_t* kv_offsets_host,
                                  const int32_t* kv_offsets_dev, const int32_t* sel, const int32_t* sel_offsets_host,
                                  const int32_t* sel_offsets_dev, const void* w_uv, float scale, float* out,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  AbsorbedLaunch q{};
  int st = sparse_prepare(g, B, L, q_lat, q_pe, c_kv, k_pe, kv_offsets_host, kv_offsets_dev, sel, sel_offsets_host,
                          sel_offsets_dev, w_uv, scale, out, workspace, workspace_bytes, &q);
  if (st) return st;
  hipStream_t s = (hipStream_t)stream;
  if ((st = hip_status(absorbed_attn_sparse(q, sel, kv_offsets_dev, kv_offsets_host[0],
                                            kv_offsets_host[1] - kv_offsets_host[0], s))))
    return st;
  return hip_status(combine_upproj(q, kBF16, out, s));
}

int mla_absorbed_attention_sparse_fp8(const mla_geom* g, int32_t B, int32_t L, const void* q_lat, const void* q_pe,
                                      const void* codes, const float* scales, const int32_t* kv_offsets_host,
                                      const int32_t* kv_offsets_dev, const int32_t* sel,
                                      const int32_t* sel_offsets_host, const int32_t* sel_offsets_dev,
                                      const void* w_uv, float scale, float* out, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (!codes || !scales) return MLA_E_NULL;
  AbsorbedLaunch q{};
  int st = sparse_prepare(g, B, L, q_lat, q_pe, codes, codes, kv_offsets_host, kv_offsets_dev, sel, sel_offsets_host,
                          sel_offsets_dev, w_uv, scale, out, workspace, workspace_bytes, &q);
  if (st) return st;
  hipStream_t s = (hipStream_t)stream;
  if ((st = hip_status(absorbed_attn_sparse_fp8(q, codes, scales, sel, kv_offsets_dev, kv_offsets_host[0],
                                                kv_offsets_host[1] - kv_offsets_host[0], s))))
    return st;
  return hip_status(combine_upproj(q, kBF16, out, s));
}

int mla_materialize_kv(const mla_geom* g, mla_dtype dt, int64_t T, const void* c_kv, const void* k_pe,
                       const void* w_uk, const void* w_uv, void* k, void* v, void* stream) {
  int st = check_geom(g);
  if (st) return st;
  if (!dtype_ok(dt)) return MLA_E_UNSUPPORTED;
  if (T < 1 || T > INT32_MAX) return MLA_E_SHAPE;
  if (!c_kv || !w_uk || !w_uv || !k || !v) return MLA_E_NULL;
  if (g->rope > 0 && !k_pe) return MLA_E_NULL;
  if (dt == MLA_BF16 && (g->r % 64 != 0 || g->n % 64 != 0 || g->v % 64 != 0 || g->rope % 8 != 0))
    return MLA_E_UNSUPPORTED;
  return hip_status(materialize_kv(dt == MLA_BF16 ? kBF16 : kF32, T, g->heads, g->r, g->n, g->v, g->rope, c_kv,
                                   k_pe, w_uk, w_uv, k, v, (hipStream_t)stream));
}

int mla_materialized_workspace_size(const mla_geom* g, mla_dtype dt, int32_t B, int32_t L,
                                    const int32_t* kv_offsets_host, size_t* bytes_out) {
  int st = check_geom(g);
  if (st) return st;
  if (!dtype_ok(dt)) return MLA_E_UNSUPPORTED;
  if (!bytes_out) return MLA_E_NULL;
  if ((st = check_offsets(B, L, kv_offsets_host))) return st;
  if ((int64_t)L * g->heads > INT32_MAX / 64) return MLA_E_SHAPE;
  if ((st = materialized_supported(g, dt))) return st;
  SplitPlan p{};
  if ((st = make_plan(B, L, g->heads, kv_offsets_host, L, g->heads, g->v, 4, dt == MLA_BF16, &p))) return st;
  *bytes_out = p.ws_bytes;
  return MLA_OK;
}

int mla_materialized_attention(const mla_geom* g, mla_dtype dt, int32_t B, int32_t L, const void* q_nope,
                               const void* q_pe, const void* k, const void* v, const int32_t* kv_offsets_host,
                               const int32_t* kv_offsets_dev, float scale, float* out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  int st = check_geom(g);
  if (st) return st;
  if (!dtype_ok(dt)) return MLA_E_UNSUPPORTED;
  if ((st = check_offsets(B, L, kv_offsets_host))) return st;
  if ((int64_t)L * g->heads > INT32_MAX / 64) return MLA_E_SHAPE;
  if (!q_nope || !k || !v || !kv_offsets_dev || !out) return MLA_E_NULL;
  if (g->rope > 0 && !q_pe) return MLA_E_NULL;
  if (g->n < 1) return MLA_E_SHAPE;
  if ((st = materialized_supported(g, dt))) return st;
  SplitPlan p{};
  if ((st = make_plan(B, L, g->heads, kv_offsets_host, L, g->heads, g->v, 4, dt == MLA_BF16, &p))) return st;
  if (!workspace || workspace_bytes < p.ws_bytes) return MLA_E_WORKSPACE;
  MaterializedLaunch q{};
  q.n = g->n; q.rope = g->rope; q.v_dim = g->v; q.H = g->heads; q.B = B; q.L = L;
  q.q_nope = q_nope; q.q_pe = q_pe; q.k = k; q.v = v;
  q.off_dev = kv_offsets_dev; q.scale = scale;
  q.off0 = kv_offsets_host[0]; q.kv1 = kv_offsets_host[1] - kv_offsets_host[0];
  q.ws_o = workspace;
  q.ws_ml = (float*)((char*)workspace + align_up(p.ws_o_bytes));
  q.plan = p;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = (dt == MLA_BF16) ? materialized_attn_bf16(q, s) : attn_f32(nullptr, &q, s);
  if (e != hipSuccess) return MLA_E_HIP;
  return hip_status(combine_materialized(q, dt == MLA_BF16 ? kBF16 : kF32, out, s));
}


// ---- pooled top-k indexer ------------------------------------------------------
namespace {
constexpr int kPoolWindow = 4;
constexpr int32_t kPoolReady = 1;   // mla_pool.valid: every covered window is pooled
constexpr int32_t kPoolStale = 2;   // mla_pool.valid: a trim cut a window (a step must run before scores)
// The fused step pools the tail windows on one workgroup per sequence: used
// only while the tail is short, else the pooling kernel spreads it out.
constexpr int64_t kFusedTailWindows = 16;
constexpr int32_t kFixedMaxTokens = 16;   // fixed-capacity update lists: steps of at most this many tokens
int64_t pool_windows(int64_t T) { return (T + kPoolWindow - 1) / kPoolWindow; }

// offsets: off[0] >= 0, non-decreasing, every Kv_b >= min_len
int check_plain_offsets(int32_t B, const int32_t* off, int64_t min_len) {
  if (!off) return MLA_E_NULL;
  if (B < 1 || off[0] < 0) return MLA_E_SHAPE;
  for (int32_t b = 0; b < B; ++b)
    if ((int64_t)off[b + 1] - off[b] < min_len) return MLA_E_SHAPE;
  return MLA_OK;
}

bool pool_guards_hold(const mla_pool* pool, int32_t B, int32_t d, const int32_t* off, int32_t S, int32_t padded) {
  if (!pool->valid) return false;                              // the cache has a pool
  if (padded) return false;                                    // there is no padding
  if (pool->batch != B || pool->d != d) return false;          // the batch shape matches
  for (int32_t b = 0; b < B; ++b)                              // the cache is as long as remembered
    if ((int64_t)pool->lengths[b] != (int64_t)off[b + 1] - off[b] - S) return false;
  return true;
}
}  // namespace

int mla_indexer_pool_init(mla_pool* pool, float* pooled, int32_t capacity, int32_t batch_max, int32_t* lengths) {
  if (!pool || !pooled || !lengths) return MLA_E_NULL;
  if (capacity < 1 || batch_max < 1) return MLA_E_SHAPE;
  pool->pooled = pooled;
  pool->capacity = capacity;
  pool->batch_max = batch_max;
  pool->batch = 0;
  pool->d = 0;
  pool->valid = 0;
  pool->lengths = lengths;
  for (int32_t b = 0; b < batch_max; ++b) lengths[b] = 0;
  return MLA_OK;
}

int mla_indexer_pool_plan(const mla_pool* pool, int32_t B, int32_t d, const int32_t* kv_offsets_host, int32_t S,
                          int32_t padded, int32_t* incremental_out) {
  if (!pool || !incremental_out || !pool->lengths) return MLA_E_NULL;
  if (S < 1) return MLA_E_SHAPE;
  int st = check_plain_offsets(B, kv_offsets_host, S);
  if (st) return st;
  if (B > pool->batch_max) return MLA_E_SHAPE;
  *incremental_out = pool_guards_hold(pool, B, d, kv_offsets_host, S, padded) ? 1 : 0;
  return MLA_OK;
}

int mla_indexer_pool_step(mla_pool* pool, int32_t B, int32_t d, const void* keys, int64_t key_stride,
                          const int32_t* kv_offsets_host, const int32_t* kv_offsets_dev, int32_t S, int32_t padded,
                          int32_t* incremental_out, void* stream) {
  if (!pool || !pool->pooled || !pool->lengths || !keys || !kv_offsets_dev) return MLA_E_NULL;
  if (S < 1 || key_stride < d) return MLA_E_SHAPE;
  int st = check_plain_offsets(B, kv_offsets_host, S);
  if (st) return st;
  if (B > pool->batch_max) return MLA_E_SHAPE;
  if (d < 8 || d > 1024 || d % 8 != 0) return MLA_E_UNSUPPORTED;
  const bool inc = pool_guards_hold(pool, B, d, kv_offsets_host, S, padded);
  int64_t wmax = 0;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t kv = (int64_t)kv_offsets_host[b + 1] - kv_offsets_host[b];
    if (pool_windows(kv) > pool->capacity) return MLA_E_SHAPE;
    const int64_t first = inc ? (kv - S) / kPoolWindow : 0;
    wmax = std::max(wmax, pool_windows(kv) - first);
  }
  if ((int64_t)kv_offsets_host[B] * key_stride > INT64_MAX / 2) return MLA_E_SHAPE;
  pool->valid = 0;   // until the launch is known to be enqueued
  st = hip_status(indexer_pool(keys, key_stride, kv_offsets_dev, B, d, S, !inc, (int)wmax, pool->pooled,
                               pool->capacity, (hipStream_t)stream));
  if (st) return st;
  for (int32_t b = 0; b < B; ++b) pool->lengths[b] = kv_offsets_host[b + 1] - kv_offsets_host[b];
  pool->batch = B;
  pool->d = d;
  pool->valid = kPoolReady;
  if (incremental_out) *incremental_out = inc ? 1 : 0;
  return MLA_OK;
}

int mla_indexer_update_list(int32_t first, int32_t windows, int32_t complete, int32_t S, int32_t target,
                            int32_t* list_out, int32_t* capacity_out) {
  if (!list_out || !capacity_out) return MLA_E_NULL;
  if (first < 0 || windows < first || complete < 0 || complete > windows || first > complete || S < 0 ||
      !(target == 8 || target == 16))
    return MLA_E_SHAPE;
  const int32_t nd = windows - first;                  // real updates: windows first .. windows - 1
  int32_t C = std::max<int32_t>(1, nd);
  int32_t n = 0;
  for (int32_t w = first; w < windows; ++w) list_out[n++] = w;
  if (S <= kFixedMaxTokens && C <= target && complete >= target) C = target;
  if (n == 0) list_out[n++] = complete > 0 ? 0 : windows - 1;   // an empty update still has one row
  // fillers: the complete windows in order whose destinations are not in the list
  for (int32_t w = 0; w < complete && n < C; ++w) {
    bool used = false;
    for (int32_t k = 0; k < n; ++k) used = used || list_out[k] == w;
    if (!used) list_out[n++] = w;
  }
  *capacity_out = C;
  return n == C ? MLA_OK : MLA_E_SHAPE;
}

int mla_indexer_pool_step_fixed(mla_pool* pool, int32_t B, int32_t d, const void* keys, int64_t key_stride,
                                const int32_t* kv_offsets_host, const int32_t* kv_offsets_dev, int32_t S,
                                int32_t padded, int32_t target, int32_t* incremental_out, int32_t* capacity_out,
                                void* stream) {
  if (!pool || !pool->pooled || !pool->lengths || !keys || !kv_offsets_dev) return MLA_E_NULL;
  if (S < 1 || key_stride < d || !(target == 8 || target == 16)) return MLA_E_SHAPE;
  int st = check_plain_offsets(B, kv_offsets_host, S);
  if (st) return st;
  if (B > pool->batch_max) return MLA_E_SHAPE;
  if (d < 8 || d > 1024 || d % 8 != 0) return MLA_E_UNSUPPORTED;
  bool fixed = pool_guards_hold(pool, B, d, kv_offsets_host, S, padded) && S <= kFixedMaxTokens;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t kv = (int64_t)kv_offsets_host[b + 1] - kv_offsets_host[b];
    if (pool_windows(kv) > pool->capacity) return MLA_E_SHAPE;
    const int64_t nd = pool_windows(kv) - (kv - S) / kPoolWindow;
    fixed = fixed && nd <= target && kv / kPoolWindow >= target;
  }
  if ((int64_t)kv_offsets_host[B] * key_stride > INT64_MAX / 2) return MLA_E_SHAPE;
  if (!fixed) {   // the ordinary step, with its own shape
    if (capacity_out) *capacity_out = 0;
    return mla_indexer_pool_step(pool, B, d, keys, key_stride, kv_offsets_host, kv_offsets_dev, S, padded,
                                 incremental_out, stream);
  }
  pool->valid = 0;   // until the launch is known to be enqueued
  st = hip_status(indexer_pool_fixed(keys, key_stride, kv_offsets_dev, B, d, S, target, pool->pooled,
                                     pool->capacity, (hipStream_t)stream));
  if (st) return st;
  for (int32_t b = 0; b < B; ++b) pool->lengths[b] = kv_offsets_host[b + 1] - kv_offsets_host[b];
  pool->batch = B;
  pool->d = d;
  pool->valid = kPoolReady;
  if (incremental_out) *incremental_out = 1;
  if (capacity_out) *capacity_out = target;
  return MLA_OK;
}

int mla_indexer_pool_trim(mla_pool* pool, int32_t B, const int32_t* new_lengths) {
  if (!pool || !new_lengths || !pool->lengths) return MLA_E_NULL;
  if (!pool->valid || B != pool->batch) return MLA_E_SHAPE;
  for (int32_t b = 0; b < B; ++b)
    if (new_lengths[b] < 0) return MLA_E_SHAPE;
  // A cut inside a window leaves that window's pooled key holding rows past the
  // cut: the pool may seed the next step (which recomputes from that window on)
  // but must not be scored until a step has run.
  bool stale = false;
  for (int32_t b = 0; b < B; ++b) {
    if (new_lengths[b] < pool->lengths[b]) {
      if (new_lengths[b] % kPoolWindow != 0) stale = true;
      pool->lengths[b] = new_lengths[b];
    }
  }
  if (stale) pool->valid = kPoolStale;
  return MLA_OK;
}

int mla_indexer_scores(const mla_pool* pool, int32_t B, const float* q, const int32_t* kv_offsets_host,
                       const int32_t* kv_offsets_dev, float* scores, void* stream) {
  if (!pool || !pool->pooled || !pool->lengths || !q || !kv_offsets_dev || !scores) return MLA_E_NULL;
  int st = check_plain_offsets(B, kv_offsets_host, 1);
  if (st) return st;
  if (pool->valid != kPoolReady || B != pool->batch) return MLA_E_SHAPE;   // a trim cut a window: step first
  int64_t wmax = 0;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t kv = (int64_t)kv_offsets_host[b + 1] - kv_offsets_host[b];
    if (pool->lengths[b] != kv) return MLA_E_SHAPE;   // the pool must cover the cache as it is
    wmax = std::max(wmax, pool_windows(kv));
  }
  return hip_status(indexer_scores(pool->pooled, pool->capacity, pool->d, q, kv_offsets_dev, B, (int)wmax, scores,
                                   nullptr, 0, 0, (hipStream_t)stream));
}

int mla_indexer_pool_step_scores(mla_pool* pool, int32_t B, int32_t d, const void* keys, int64_t key_stride,
                                 const int32_t* kv_offsets_host, const int32_t* kv_offsets_dev, int32_t S,
                                 int32_t padded, const float* q, float* scores, int32_t* incremental_out,
                                 void* stream) {
  if (!pool || !pool->pooled || !pool->lengths || !keys || !kv_offsets_dev || !q || !scores) return MLA_E_NULL;
  if (S < 1 || key_stride < d) return MLA_E_SHAPE;
  int st = check_plain_offsets(B, kv_offsets_host, S);
  if (st) return st;
  if (B > pool->batch_max) return MLA_E_SHAPE;
  if (d < 8 || d > 1024 || d % 8 != 0) return MLA_E_UNSUPPORTED;
  const bool inc = pool_guards_hold(pool, B, d, kv_offsets_host, S, padded);
  int64_t wmax = 0, tail_max = 0;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t kv = (int64_t)kv_offsets_host[b + 1] - kv_offsets_host[b];
    if (pool_windows(kv) > pool->capacity) return MLA_E_SHAPE;
    wmax = std::max(wmax, pool_windows(kv));
    tail_max = std::max(tail_max, pool_windows(kv) - (kv - S) / kPoolWindow);
  }
  if ((int64_t)kv_offsets_host[B] * key_stride > INT64_MAX / 2) return MLA_E_SHAPE;
  pool->valid = 0;   // until the launches are known to be enqueued
  hipStream_t hs = (hipStream_t)stream;
  if (inc && tail_max <= kFusedTailWindows) {   // one launch: the scoring pools the tail windows itself
    st = hip_status(indexer_scores(pool->pooled, pool->capacity, d, q, kv_offsets_dev, B, (int)wmax, scores,
                                   (const uint16_t*)keys, key_stride, S, hs));
  } else {   // every window, or a long tail spread over the pooling kernel's workgroups; then score
    st = hip_status(indexer_pool(keys, key_stride, kv_offsets_dev, B, d, S, !inc, (int)(inc ? tail_max : wmax),
                                 pool->pooled, pool->capacity, hs));
    if (!st)
      st = hip_status(indexer_scores(pool->pooled, pool->capacity, d, q, kv_offsets_dev, B, (int)wmax, scores,
                                     nullptr, 0, 0, hs));
  }
  if (st) return st;
  for (int32_t b = 0; b < B; ++b) pool->lengths[b] = kv_offsets_host[b + 1] - kv_offsets_host[b];
  pool->batch = B;
  pool->d = d;
  pool->valid = kPoolReady;
  if (incremental_out) *incremental_out = inc ? 1 : 0;
  return MLA_OK;
}

int mla_indexer_selection_offsets(int32_t B, const int32_t* kv_offsets_host, int32_t budget,
                                  int32_t* sel_offsets_out) {
  if (!sel_offsets_out) return MLA_E_NULL;
  if (budget < 1) return MLA_E_SHAPE;
  int st = check_plain_offsets(B, kv_offsets_host, 1);
  if (st) return st;
  int64_t acc = 0;
  for (int32_t b = 0; b < B; ++b) acc += std::min<int64_t>(budget, (int64_t)kv_offsets_host[b + 1] - kv_offsets_host[b]);
  if (acc > INT32_MAX) return MLA_E_SHAPE;
  sel_offsets_out[0] = 0;
  for (int32_t b = 0; b < B; ++b)
    sel_offsets_out[b + 1] =
        sel_offsets_out[b] + (int32_t)std::min<int64_t>(budget, (int64_t)kv_offsets_host[b + 1] - kv_offsets_host[b]);
  return MLA_OK;
}

int mla_indexer_select(int32_t B, const float* scores, int32_t capacity, const int32_t* kv_offsets_host,
                       const int32_t* kv_offsets_dev, int32_t budget, const int32_t* sel_offsets_dev, int32_t* sel,
                       void* stream) {
  if (!scores || !kv_offsets_dev || !sel_offsets_dev || !sel) return MLA_E_NULL;
  if (budget < 1 || capacity < 1) return MLA_E_SHAPE;
  int st = check_plain_offsets(B, kv_offsets_host, 1);
  if (st) return st;
  for (int32_t b = 0; b < B; ++b)
    if (pool_windows((int64_t)kv_offsets_host[b + 1] - kv_offsets_host[b]) > capacity) return MLA_E_SHAPE;
  return hip_status(indexer_select(scores, capacity, kv_offsets_dev, B, budget, sel_offsets_dev, sel,
                                   (hipStream_t)stream));
}

}  // extern "C"
