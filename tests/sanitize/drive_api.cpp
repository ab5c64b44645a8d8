// drive_api.cpp -- drives every entry point of the C ABI (include/mla.h) on the
// host, against the launcher stand-ins of launch_stub.cpp: valid calls (which
// reach a stand-in) and invalid ones (which must fail validation), over random
// and extreme sizes.  Built with -fsanitize=address,undefined; any report or a
// failed check ends the program with a non-zero status.
#include "../../include/mla.h"

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <random>
#include <vector>

namespace mla { extern int stub_launches; }

static int failures = 0;
#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

static void* fake(uintptr_t x) { return reinterpret_cast<void*>(x); }   // never dereferenced on the host

static std::vector<int32_t> offsets(const std::vector<int64_t>& lens) {
  std::vector<int32_t> o(lens.size() + 1, 0);
  for (size_t i = 0; i < lens.size(); ++i) o[i + 1] = (int32_t)(o[i] + lens[i]);
  return o;
}

int main() {
  std::mt19937_64 rng(20261202);
  auto uni = [&](int64_t lo, int64_t hi) { return std::uniform_int_distribution<int64_t>(lo, hi)(rng); };
  for (int s = -7; s <= 1; ++s) CHECK(mla_status_string(s) != nullptr);
  CHECK(mla_version() >= 1);

  // path selection over random and extreme geometries
  for (int it = 0; it < 20000; ++it) {
    mla_geom g{(int32_t)uni(1, 4096), (int32_t)uni(0, 4096), (int32_t)uni(0, 4096), (int32_t)uni(0, 128), 1};
    if (it % 97 == 0) g = mla_geom{std::numeric_limits<int32_t>::max(), std::numeric_limits<int32_t>::max(),
                                   std::numeric_limits<int32_t>::max(), 0, 1};
    const int64_t T = it % 3 == 0 ? 0 : uni(1, it % 11 == 0 ? std::numeric_limits<int64_t>::max() : 1 << 20);
    const int64_t L = T == 0 ? uni(1, 1 << 20) : uni(1, T);
    int32_t path = -1;
    int64_t m = -1;
    CHECK(mla_select_path(&g, L, T, &path, &m) == MLA_OK);
    CHECK(m >= 1 && (path == MLA_ABSORBED) == (L <= m));
  }
  {
    mla_geom g{512, 128, 128, 64, 128};
    int32_t path;
    CHECK(mla_select_path(&g, 0, 0, &path, nullptr) == MLA_E_SHAPE);
    CHECK(mla_select_path(&g, 9, 8, &path, nullptr) == MLA_E_SHAPE);
    CHECK(mla_select_path(nullptr, 1, 0, &path, nullptr) == MLA_E_NULL);
  }

  // draft cap
  for (int it = 0; it < 2000; ++it) {
    const int n = (int)uni(1, 24);
    std::vector<double> c(n), by(n);
    for (auto& x : c) x = 0.1 + (double)uni(0, 1000) / 100.0;
    int32_t cap = -1;
    double sp = 0.0;
    CHECK(mla_draft_cap(c.data(), n, (double)uni(0, 100) / 100.0, (double)uni(0, 50) / 100.0, &cap, &sp,
                        by.data()) == MLA_OK);
    CHECK(cap >= 0 && cap < n && sp >= 1.0);
  }
  {
    double c[2] = {1.0, -1.0};
    int32_t cap;
    double sp;
    CHECK(mla_draft_cap(c, 2, 0.5, 0.1, &cap, &sp, nullptr) == MLA_E_SHAPE);
    CHECK(mla_draft_cap(c, 0, 0.5, 0.1, &cap, &sp, nullptr) == MLA_E_SHAPE);
  }

  // attention planning and launches (stand-ins) over random batches, both dtypes
  const mla_geom geoms[] = {{512, 128, 128, 64, 128}, {512, 192, 256, 64, 32}, {512, 256, 256, 64, 64},
                            {512, 128, 128, 0, 16}, {256, 64, 64, 32, 4}};
  for (int it = 0; it < 3000; ++it) {
    const mla_geom g = geoms[it % 5];
    const mla_dtype dt = (it / 5) % 2 ? MLA_BF16 : MLA_F32;
    const int32_t B = (int32_t)uni(1, it % 7 == 0 ? 300 : 8);
    const int32_t L = (int32_t)uni(1, it % 13 == 0 ? 2048 : 16);
    std::vector<int64_t> lens(B);
    for (auto& x : lens) x = uni(L, it % 17 == 0 ? (1 << 22) + 64 : 40000);
    const auto off = offsets(lens);
    size_t ws = 0;
    const int st = mla_absorbed_workspace_size(&g, dt, B, L, off.data(), &ws);
    if (st == MLA_OK) {
      const int before = mla::stub_launches;
      CHECK(mla_absorbed_attention(&g, dt, B, L, fake(64), fake(64), fake(64), fake(64), off.data(), (int32_t*)fake(64),
                                   fake(64), 0.1f, (float*)fake(64), fake(256), ws, nullptr) == MLA_OK);
      CHECK(mla::stub_launches == before + 2);
      CHECK(mla_absorbed_attention(&g, dt, B, L, fake(64), fake(64), fake(64), fake(64), off.data(), (int32_t*)fake(64),
                                   fake(64), 0.1f, (float*)fake(64), fake(256), ws - 1, nullptr) == MLA_E_WORKSPACE);
      CHECK(mla_absorbed_splits(&g, dt, B, L, fake(64), fake(64), fake(64), fake(64), off.data(), (int32_t*)fake(64),
                                0.1f, fake(256), ws, nullptr) == MLA_OK);
      CHECK(mla_absorbed_merge(&g, dt, B, L, off.data(), (int32_t*)fake(64), fake(64), (float*)fake(64), fake(256), ws,
                               nullptr) == MLA_OK);
      if (dt == MLA_BF16) {
        CHECK(mla_absorbed_attention_fp8(&g, B, L, fake(64), fake(64), fake(64), (float*)fake(64), off.data(),
                                         (int32_t*)fake(64), fake(64), 0.1f, (float*)fake(64), fake(256), ws,
                                         nullptr) == (g.r == 512 ? MLA_OK : MLA_E_UNSUPPORTED));
        CHECK(mla_absorbed_attention_fp8q(&g, B, L, fake(64), fake(64), (float*)fake(64), off.data(),
                                          (int32_t*)fake(64), fake(64), 0.1f, (float*)fake(64), fake(256), ws,
                                          nullptr) == (g.r == 512 ? MLA_OK : MLA_E_UNSUPPORTED));
        size_t qb = 0;
        CHECK(mla_query_fp8_bytes(&g, B, L, &qb) == MLA_OK);
        CHECK(qb == (size_t)B * (size_t)(((int64_t)L * g.heads + 31) / 32) * 19456);
      }
    } else {
      CHECK(st == MLA_E_UNSUPPORTED || st == MLA_E_SHAPE);
    }
    size_t wm = 0;
    const int sm = mla_materialized_workspace_size(&g, dt, B, L, off.data(), &wm);
    if (sm == MLA_OK) {
      CHECK(mla_materialized_attention(&g, dt, B, L, fake(64), fake(64), fake(64), fake(64), off.data(),
                                       (int32_t*)fake(64), 0.1f, (float*)fake(64), fake(256), wm, nullptr) == MLA_OK);
    }
    // selections: budget-limited, at least one position each
    std::vector<int64_t> klen(B);
    for (int32_t b = 0; b < B; ++b) klen[b] = std::min<int64_t>(lens[b], uni(1, 4096));
    const auto soff = offsets(klen);
    size_t wsp = 0;
    if (dt == MLA_BF16 && mla_absorbed_sparse_workspace_size(&g, B, L, off.data(), soff.data(), &wsp) == MLA_OK) {
      CHECK(mla_absorbed_attention_sparse(&g, B, L, fake(64), fake(64), fake(64), fake(64), off.data(),
                                          (int32_t*)fake(64), (int32_t*)fake(64), soff.data(), (int32_t*)fake(64),
                                          fake(64), 0.1f, (float*)fake(64), fake(256), wsp, nullptr) ==
            (g.r == 512 ? MLA_OK : MLA_E_UNSUPPORTED));
    }
  }
  {
    // malformed offsets and sizes are refused before any launch
    const mla_geom g{512, 128, 128, 64, 128};
    const int before = mla::stub_launches;
    std::vector<int32_t> bad = {0, 5, 3};
    size_t ws;
    CHECK(mla_absorbed_workspace_size(&g, MLA_BF16, 2, 4, bad.data(), &ws) == MLA_E_SHAPE);
    std::vector<int32_t> neg = {-4, 10};
    CHECK(mla_absorbed_workspace_size(&g, MLA_BF16, 1, 4, neg.data(), &ws) == MLA_E_SHAPE);
    std::vector<int32_t> ok = {0, 100};
    CHECK(mla_absorbed_workspace_size(&g, MLA_BF16, 1, 0, ok.data(), &ws) == MLA_E_SHAPE);
    CHECK(mla_absorbed_workspace_size(&g, MLA_BF16, 0, 4, ok.data(), &ws) == MLA_E_SHAPE);
    CHECK(mla_absorbed_workspace_size(nullptr, MLA_BF16, 1, 4, ok.data(), &ws) == MLA_E_NULL);
    CHECK(mla_absorbed_workspace_size(&g, (mla_dtype)7, 1, 4, ok.data(), &ws) == MLA_E_UNSUPPORTED);
    CHECK(mla_fold_query(&g, MLA_BF16, 0, fake(64), fake(64), fake(64), nullptr) == MLA_E_SHAPE);
    CHECK(mla_materialize_kv(&g, MLA_BF16, 0, fake(64), fake(64), fake(64), fake(64), fake(64), fake(64), nullptr) ==
          MLA_E_SHAPE);
    CHECK(mla_quantize_latent_fp8(&g, 0, fake(64), fake(64), fake(64), (float*)fake(64), nullptr) == MLA_E_SHAPE);
    CHECK(mla::stub_launches == before);
    CHECK(mla_fold_query(&g, MLA_BF16, 8, fake(64), fake(64), fake(64), nullptr) == MLA_OK);
    CHECK(mla_materialize_kv(&g, MLA_BF16, 8192, fake(64), fake(64), fake(64), fake(64), fake(64), fake(64),
                             nullptr) == MLA_OK);
    CHECK(mla_quantize_latent_fp8(&g, 8192, fake(64), fake(64), fake(64), (float*)fake(64), nullptr) == MLA_OK);
    CHECK(mla_fold_query_fp8(&g, 0, 8, fake(64), fake(64), fake(64), nullptr, fake(64), nullptr) == MLA_E_SHAPE);
    CHECK(mla_fold_query_fp8(&g, 1, 8, fake(64), fake(64), nullptr, nullptr, fake(64), nullptr) == MLA_E_NULL);
    CHECK(mla_fold_query_fp8(&g, 1, 8, fake(64), fake(64), fake(64), nullptr, fake(64), nullptr) == MLA_OK);
  }

  // pooled indexer: random steps, trims, scores and selections on the host state
  for (int it = 0; it < 500; ++it) {
    const int32_t bmax = (int32_t)uni(1, 6), cap = (int32_t)uni(1, 3000);
    std::vector<int32_t> lengths(bmax, -1);
    mla_pool pool;
    CHECK(mla_indexer_pool_init(&pool, (float*)fake(256), cap, bmax, lengths.data()) == MLA_OK);
    std::vector<int64_t> lens(uni(1, bmax), 0);
    const int32_t d = (int32_t)(8 * uni(1, 64));
    for (int step = 0; step < 12; ++step) {
      const int32_t S = (int32_t)uni(1, 80);
      for (auto& x : lens) x += S;
      const auto off = offsets(lens);
      const int32_t B = (int32_t)lens.size();
      int32_t inc = -1;
      const int pst = mla_indexer_pool_plan(&pool, B, d, off.data(), S, 0, &inc);
      CHECK(pst == MLA_OK);
      std::vector<float> q(1);
      const int sst = step % 2 ? mla_indexer_pool_step(&pool, B, d, fake(64), d, off.data(), (int32_t*)fake(64), S,
                                                       0, &inc, nullptr)
                               : mla_indexer_pool_step_scores(&pool, B, d, fake(64), d, off.data(), (int32_t*)fake(64),
                                                              S, 0, (float*)fake(64), (float*)fake(64), &inc, nullptr);
      bool fits = true;
      for (auto x : lens) fits = fits && (x + 3) / 4 <= cap;
      CHECK(sst == (fits ? MLA_OK : MLA_E_SHAPE));
      if (sst != MLA_OK) break;
      if (uni(0, 2) == 0) {   // a rejection cuts every sequence back
        std::vector<int32_t> nl(B);
        bool cut = false;   // some sequence shortened to a length inside a window
        for (int32_t b = 0; b < B; ++b) {
          nl[b] = (int32_t)uni(0, lens[b]);
          cut = cut || (nl[b] < lens[b] && nl[b] % 4 != 0);
          lens[b] = nl[b];
        }
        CHECK(mla_indexer_pool_trim(&pool, B, nl.data()) == MLA_OK);
        const auto o2 = offsets(lens);
        bool nonempty = true;
        for (auto x : lens) nonempty = nonempty && x >= 1;
        if (nonempty)
          CHECK(mla_indexer_scores(&pool, B, (float*)fake(64), o2.data(), (int32_t*)fake(64), (float*)fake(64),
                                   nullptr) == (cut ? MLA_E_SHAPE : MLA_OK));
      }
      std::vector<int32_t> so(B + 1);
      const int32_t budget = (int32_t)uni(1, 5000);
      CHECK(mla_indexer_selection_offsets(B, off.data(), budget, so.data()) == MLA_OK);
      CHECK(mla_indexer_select(B, (float*)fake(64), cap, off.data(), (int32_t*)fake(64), budget, (int32_t*)fake(64),
                               (int32_t*)fake(64), nullptr) == (fits ? MLA_OK : MLA_E_SHAPE));
    }
  }
  std::printf("api driver: %d stand-in launches, %d failed checks\n", mla::stub_launches, failures);
  return failures == 0 ? 0 : 1;
}
