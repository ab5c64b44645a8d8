// indexer.hip -- the pooled top-k indexer that picks the cached positions a
// sparse attention layer attends over (pages: "One guard, 110x off the verify
// step", sections "The sparse model is different" and "The same bug, one
// layer over").
//
// Keys of a sequence are pooled in windows of four positions (window w holds
// positions 4w .. 4w+3; the last window may be partial).  A window's pooled
// key is the float32 mean of the bf16 key rows it holds, summed in position
// order, so the same window always pools to the same bits however the
// positions arrived.  A step that appended S positions recomputes only the
// windows from floor((Kv - S) / 4) on (the old tail window and the new ones);
// windows completed before that cannot change, since positions only append.
// The host decides between that and a full recompute (the four guards).
//
// Scores: window w scores q . pooled[w] (float32, fixed summation order).
// Selection: every position carries its window's score; the first
// min(budget, Kv) positions in the order (score descending, position
// ascending) are written in increasing position order.  A histogram over
// 2048 equal slices of the score range finds the slice holding the
// budget-th position; inside that slice a direct count (up to 64 windows) or a
// weighted radix select (8-bit digits of the score's order key, weight =
// positions in the window) finds the score of the last window taken, and a
// scan over windows in index order then places each taken window's positions.
// Integer work only after the scores: the selection of given scores is exact.

#include "mla_device.h"
#include "internal.h"

namespace mla {

constexpr int kWin = 4;

__device__ __forceinline__ int windows_of(int T) { return (T + kWin - 1) / kWin; }

// ---- pooling ----------------------------------------------------------------
// One wave pools window w of a sequence (rows src .. src + (n - 1) ld, n <= 4)
// into dst: lane l takes the 8-column chunks l, l + 64, ...; rows are summed in
// position order in float32, then divided by n (correctly rounded).
__device__ __forceinline__ void pool_one_window(const uint16_t* __restrict__ src, long long ld, int n, int d,
                                                float* __restrict__ dst) {
  const int lane = threadIdx.x & 63;
  const float fn = (float)n;
  for (int c = lane; c < d / 8; c += kWave) {
    float acc[8];
    const u32x4 r0 = ld16(src + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] = bf16_lo(r0[e]);
      acc[2 * e + 1] = bf16_hi(r0[e]);
    }
    for (int j = 1; j < n; ++j) {
      const u32x4 r = ld16(src + (long long)j * ld + 8 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += bf16_lo(r[e]);
        acc[2 * e + 1] += bf16_hi(r[e]);
      }
    }
    f32x4 m0, m1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      m0[e] = acc[e] / fn;       // correctly rounded division (exact for n = 1, 2, 4)
      m1[e] = acc[4 + e] / fn;
    }
    *reinterpret_cast<f32x4*>(dst + 8 * c) = m0;
    *reinterpret_cast<f32x4*>(dst + 8 * c + 4) = m1;
  }
}

// grid (ceil(wmax / 4), B), 256 threads: one wave per window
__global__ __launch_bounds__(256) void pool_windows_kernel(const uint16_t* __restrict__ keys, long long ld,
                                                           const int32_t* __restrict__ off, int d, int S, int full,
                                                           float* __restrict__ pooled, int cap) {
  const int b = blockIdx.y;
  const int o0 = off[b];
  const int Kv = off[b + 1] - o0;
  const int first = full ? 0 : (Kv - S) / kWin;
  const int w = first + blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= windows_of(Kv)) return;
  pool_one_window(keys + ((long long)o0 + kWin * w) * ld, ld, min(kWin, Kv - kWin * w), d,
                  pooled + ((long long)b * cap + w) * d);
}

// The fixed-capacity update list ("Over 107 tok/s Qwen3.8-Flash-Next on M3
// Ultra", section "Why doing eight rows can beat doing two"): every sequence
// recomputes exactly P windows, its real updates (windows first .. W - 1, the
// old tail window and the new ones) followed by fillers, the complete windows
// 0, 1, ... (all before first, so their destinations are distinct from the real
// ones), whose rows have not changed: a filler writes back the bits already
// stored.  The host launches this only where every sequence has at most P real
// updates and at least P complete windows.  grid (P / 4, B): one wave per slot.
__global__ __launch_bounds__(256) void pool_fixed_kernel(const uint16_t* __restrict__ keys, long long ld,
                                                         const int32_t* __restrict__ off, int d, int S,
                                                         float* __restrict__ pooled, int cap) {
  const int b = blockIdx.y;
  const int o0 = off[b];
  const int Kv = off[b + 1] - o0;
  const int first = (Kv - S) / kWin;
  const int nd = windows_of(Kv) - first;              // real updates
  const int c = blockIdx.x * 4 + (threadIdx.x >> 6);  // slot of the list
  const int w = c < nd ? first + c : c - nd;
  pool_one_window(keys + ((long long)o0 + kWin * w) * ld, ld, min(kWin, Kv - kWin * w), d,
                  pooled + ((long long)b * cap + w) * d);
}

// ---- scores -----------------------------------------------------------------
// grid (min(ceil(wmax / 16), max(1, 512 / B)) [+ 1 with TAIL], B), 256 threads:
// group x of a sequence is windows 4x .. 4x + 3; lane l takes the float4 chunks
// l, l + 64, ...
constexpr int kScoreWin = 4;      // windows per wave and group (the reduction below assumes four)
constexpr int kScoreBlocks = 512;  // workgroups per launch (4 waves each), shared by the sequences
// One wave scores groups of kScoreWin consecutive windows, striding over the
// sequence's groups; the next group's loads are in flight while the current
// group is reduced.  J = 16-byte loads per lane and window (d <= 256 J).
// TAIL: the launch also pools the tail windows (from floor((Kv - S) / 4) on).
// The first workgroup of the grid (dispatched first) takes the groups that hold them: each wave
// pools its tail windows from the key rows with the pooling kernel's arithmetic
// (rows summed in position order in float32, then divided by the row count),
// stores them and scores the values it holds; the other workgroups stream the
// groups before them.
struct TailArgs {
  const uint16_t* keys;   // bf16 key rows, position p of sequence b at keys + (off[b] + p) * ld
  long long ld;
  int S;
};

template <int J, bool TAIL>
__global__ __launch_bounds__(256) void window_scores_kernel(float* __restrict__ pooled, int cap, int d,
                                                            const float* __restrict__ q,
                                                            const int32_t* __restrict__ off,
                                                            float* __restrict__ scores, TailArgs ta) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.y;
  const int Kv = off[b + 1] - off[b];
  const int W = windows_of(Kv);
  const int ngroups = (W + kScoreWin - 1) / kScoreWin;
  const int first = TAIL ? (Kv - ta.S) / kWin : W;   // windows from here on are pooled here
  const int gtail = TAIL ? min(first / kScoreWin, ngroups) : ngroups;   // first group with a tail window
  const bool tail_block = TAIL && blockIdx.x == 0;
  const int sb = (int)blockIdx.x - (TAIL ? 1 : 0);   // index among the streaming workgroups
  const int nc = d / 4;
  if (tail_block ? gtail + wave >= ngroups : sb * 4 + wave >= gtail) return;
  f32x4 qv[J];
#pragma unroll
  for (int j = 0; j < J; ++j) qv[j] = *reinterpret_cast<const f32x4*>(q + (long long)b * d + 4 * min(lane + kWave * j, nc - 1));
  const float* base = pooled + (long long)b * cap * d;
  // every load is issued unconditionally (clamped addresses, values masked at use),
  // so the wait for the current group leaves the next group's loads in flight
  auto load = [&](int grp, f32x4 (&pv)[kScoreWin][J]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kScoreWin; ++k) {
      const float* row = base + (long long)min(grp * kScoreWin + k, W - 1) * d;
#pragma unroll
      for (int j = 0; j < J; ++j) pv[k][j] = *reinterpret_cast<const f32x4*>(row + 4 * min(lane + kWave * j, nc - 1));
    }
  };
  // scores of the group's four windows from pv: fixed-order fma chains, then the four
  // reduced together (after the xor-32 and xor-16 exchanges lane l carries window
  // l >> 4 over four lanes, then four more halvings)
  auto score = [&](int grp, const f32x4 (&pv)[kScoreWin][J]) __attribute__((always_inline)) {
    float p[kScoreWin];
#pragma unroll
    for (int k = 0; k < kScoreWin; ++k) {
      p[k] = 0.f;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const bool in = lane + kWave * j < nc;
#pragma unroll
        for (int e = 0; e < 4; ++e) p[k] = fmaf(qv[j][e], in ? pv[k][j][e] : 0.f, p[k]);
      }
    }
    const bool h = (lane & 32) != 0, gbit = (lane & 16) != 0;
    float c0 = h ? p[2] : p[0], c1 = h ? p[3] : p[1];
    c0 += __shfl_xor(h ? p[0] : p[2], 32, kWave);
    c1 += __shfl_xor(h ? p[1] : p[3], 32, kWave);
    float t = gbit ? c1 : c0;
    t += __shfl_xor(gbit ? c0 : c1, 16, kWave);
#pragma unroll
    for (int dd = 8; dd >= 1; dd >>= 1) t += __shfl_xor(t, dd, kWave);
    const int w = grp * kScoreWin + (lane >> 4);
    if ((lane & 15) == 0 && w < W) scores[(long long)b * cap + w] = t;
  };

  if (TAIL && tail_block) {
    for (int g = gtail + wave; g < ngroups; g += 4) {
      f32x4 pv[kScoreWin][J];
      load(g, pv);   // windows before `first` keep their pooled keys
#pragma unroll
      for (int k = 0; k < kScoreWin; ++k) {
        const int w = g * kScoreWin + k;
        if (w < first || w >= W) continue;
        const int n = min(kWin, Kv - kWin * w);
        const float fn = (float)n;
        const uint16_t* src = ta.keys + ((long long)off[b] + kWin * w) * ta.ld;
        float* dst = pooled + ((long long)b * cap + w) * d;
#pragma unroll
        for (int j = 0; j < J; ++j) {
          const int c = min(lane + kWave * j, nc - 1);   // columns 4c .. 4c + 3
          u32x2 x[kWin];   // every row's load in flight at once (rows past n repeat the last)
#pragma unroll
          for (int r = 0; r < kWin; ++r) x[r] = *reinterpret_cast<const u32x2*>(src + (long long)min(r, n - 1) * ta.ld + 4 * c);
          float acc[4] = {bf16_lo(x[0][0]), bf16_hi(x[0][0]), bf16_lo(x[0][1]), bf16_hi(x[0][1])};
#pragma unroll
          for (int r = 1; r < kWin; ++r) {
            if (r < n) {   // rows summed in position order, as in the pooling kernel
              acc[0] += bf16_lo(x[r][0]);
              acc[1] += bf16_hi(x[r][0]);
              acc[2] += bf16_lo(x[r][1]);
              acc[3] += bf16_hi(x[r][1]);
            }
          }
          f32x4 m;
#pragma unroll
          for (int e = 0; e < 4; ++e) m[e] = acc[e] / fn;   // correctly rounded, as in the pooling kernel
          if (lane + kWave * j < nc) *reinterpret_cast<f32x4*>(dst + 4 * c) = m;
          pv[k][j] = m;
        }
      }
      score(g, pv);
    }
    return;
  }

  // streaming workgroups: groups [0, gtail), from the end backwards
  const int stride = (int)(TAIL ? gridDim.x - 1 : gridDim.x) * 4;
  int gi = sb * 4 + wave;
  int g = gtail - 1 - gi;
  f32x4 pv[kScoreWin][J];
  load(g, pv);
  for (;;) {
    const int gni = gi + stride, gn = gtail - 1 - gni;
    f32x4 pn[kScoreWin][J];
    load(gni < gtail ? gn : g, pn);   // the last round reads its own group again (from L2)
    score(g, pv);
    if (gni >= gtail) break;
#pragma unroll
    for (int k = 0; k < kScoreWin; ++k)
#pragma unroll
      for (int j = 0; j < J; ++j) pv[k][j] = pn[k][j];
    gi = gni;
    g = gn;
  }
}

// ---- selection --------------------------------------------------------------
// Unsigned key whose order is the float order of the score (-0 counts as +0).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kBuckets = 2048;
constexpr int kHistCopies = 4;      // radix histograms (waves share them round robin)
constexpr int kStage = 32768;       // window scores staged in LDS (128 KB)
constexpr int kCand = 1024;         // boundary-bucket windows kept in an LDS list
constexpr int kOutStage = kBuckets + 2 * kCand;   // selected positions gathered in LDS, then stored in order

// Exclusive scan over the block of a 64-bit value per thread (two 32-bit
// counters in the halves, neither of which can overflow); returns the block
// total through *total.  Uses sh[kSelWaves] and two barriers.
__device__ __forceinline__ uint64_t block_exscan_u64(uint64_t v, uint64_t* sh, uint64_t* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint64_t inc = v;
#pragma unroll
  for (int dd = 1; dd < kWave; dd <<= 1) {
    const uint64_t t = __shfl_up(inc, dd, kWave);
    if (lane >= dd) inc += t;
  }
  if (lane == kWave - 1) sh[wv] = inc;
  __syncthreads();
  uint64_t before = 0, all = 0;
#pragma unroll
  for (int k = 0; k < kSelWaves; ++k) {
    const uint64_t t = sh[k];
    before += k < wv ? t : 0;
    all += t;
  }
  __syncthreads();   // sh is written again by the next call
  *total = all;
  return before + inc - v;
}

// Weighted radix select over the keys that pass `keep`: 8-bit digits from the
// top; `need` (>= 1, at most the kept weight) is the rank, in weight, of the
// wanted key from the largest.  Returns that key; *need becomes its rank among
// the windows of exactly that key.  for_each(f) calls f(key, weight) for every
// candidate this thread owns.  Uses hist[kHistCopies][256] and pick[2].
template <typename ForEach>
__device__ __forceinline__ uint32_t radix_select(ForEach for_each, uint32_t* need, uint32_t (*hist)[256], uint32_t* pick) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  uint32_t prefix = 0u, mask = 0u;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int k = tid; k < kHistCopies * 256; k += kSelThreads) (&hist[0][0])[k] = 0u;
    __syncthreads();
    for_each([&](uint32_t u, uint32_t wgt) __attribute__((always_inline)) {
      if ((u & mask) == prefix) atomicAdd(&hist[wv % kHistCopies][(u >> shift) & 255u], wgt);
    });
    __syncthreads();
    if (wv == 0) {
      // lane l: digits 4l .. 4l+3; weight of larger digits = suffix over lanes
      uint32_t t[4], sum = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t x = 0u;
#pragma unroll
        for (int k = 0; k < kHistCopies; ++k) x += hist[k][4 * lane + e];
        t[e] = x;
        sum += x;
      }
      uint32_t incl = sum;   // inclusive suffix sum over lanes >= l
#pragma unroll
      for (int dd = 1; dd < kWave; dd <<= 1) {
        const uint32_t x = __shfl_down(incl, dd, kWave);
        if (lane + dd < kWave) incl += x;
      }
      uint32_t above = incl - sum;   // weight of digits above 4l + 3
#pragma unroll
      for (int e = 3; e >= 0; --e) {
        if (above < *need && *need <= above + t[e]) {
          pick[0] = (uint32_t)(4 * lane + e);
          pick[1] = above;
        }
        above += t[e];
      }
    }
    __syncthreads();
    *need -= pick[1];
    prefix |= pick[0] << shift;
    mask |= 255u << shift;
    __syncthreads();   // pick is written again by the next pass
  }
  return prefix;
}

// The same select run by one wave over a short list in LDS (cand[c] = (order key,
// weight), c < nc): no block barriers; the wave's LDS accesses complete in order.
__device__ __forceinline__ uint32_t wave_radix_list(const uint32_t (*cand)[2], uint32_t nc, uint32_t* need,
                                                    uint32_t* hist) {
  const int lane = threadIdx.x & 63;
  uint32_t prefix = 0u, mask = 0u;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    for (int k = lane; k < 256; k += kWave) hist[k] = 0u;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    for (uint32_t c = lane; c < nc; c += kWave) {
      const uint32_t u = cand[c][0];
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], cand[c][1]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    uint32_t t[4], sum = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      t[e] = hist[4 * lane + e];
      sum += t[e];
    }
    uint32_t incl = sum;   // inclusive suffix sum over lanes >= l
#pragma unroll
    for (int dd = 1; dd < kWave; dd <<= 1) {
      const uint32_t x = __shfl_down(incl, dd, kWave);
      if (lane + dd < kWave) incl += x;
    }
    uint32_t above = incl - sum, dsel = 0u, asel = 0u;
    bool hit = false;
#pragma unroll
    for (int e = 3; e >= 0; --e) {
      if (above < *need && *need <= above + t[e]) {
        hit = true;
        dsel = (uint32_t)(4 * lane + e);
        asel = above;
      }
      above += t[e];
    }
    const int src = max(__ffsll((long long)__ballot(hit)) - 1, 0);   // exactly one lane hits
    const uint32_t D = __builtin_amdgcn_readlane(dsel, src);
    *need -= __builtin_amdgcn_readlane(asel, src);
    prefix |= D << shift;
    mask |= 255u << shift;
  }
  return prefix;
}

// The same select for a list of at most one candidate per lane: lane i counts the
// weight above and equal to its own key directly.
__device__ __forceinline__ uint32_t wave_rank_list(const uint32_t (*cand)[2], uint32_t nc, uint32_t* need) {
  const uint32_t lane = threadIdx.x & 63;
  const bool has = lane < nc;
  const uint32_t ui = has ? cand[lane][0] : 0u;
  uint32_t above = 0u, equal = 0u;
#pragma unroll 4
  for (uint32_t j = 0; j < nc; ++j) {   // the same entry for every lane: one broadcast read
    const uint32_t uj = cand[j][0], cj = cand[j][1];
    above += uj > ui ? cj : 0u;
    equal += uj == ui ? cj : 0u;
  }
  const bool hit = has && above < *need && *need <= above + equal;   // the lanes of one key
  const int src = max(__ffsll((long long)__ballot(hit)) - 1, 0);
  *need -= __builtin_amdgcn_readlane(above, src);
  return __builtin_amdgcn_readlane(ui, src);
}

// grid B, 1024 threads: one block per sequence.
__global__ __launch_bounds__(kSelThreads) void select_positions_kernel(const float* __restrict__ scores, int cap,
                                                                       const int32_t* __restrict__ off, int budget,
                                                                       const int32_t* __restrict__ sel_off,
                                                                       int32_t* __restrict__ sel) {
  __shared__ uint32_t hist[kHistCopies][256];
  // bucket histogram, then the candidate list (order key, weight) of the windows in
  // the boundary bucket; at the end the first kOutStage selected positions
  __shared__ uint32_t aux[kBuckets + 2 * kCand];
  uint32_t* const bhist = aux;
  uint32_t (*const cand)[2] = reinterpret_cast<uint32_t (*)[2]>(aux + kBuckets);
  __shared__ float sk[kStage + kStage / 32];   // window scores, one pad word after each thread's chunk
  __shared__ uint64_t scan_sh[kSelWaves];
  __shared__ float mm[2][kSelWaves];
  __shared__ uint32_t pick[2], ncand;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) {
    pick[0] = pick[1] = 0u;
    ncand = 0u;
  }
  const int b = blockIdx.x;
  const int Kv = off[b + 1] - off[b];
  int32_t* out = sel + sel_off[b];
  if (Kv <= budget) {   // every position is taken
    for (int t = tid; t < Kv; t += kSelThreads) out[t] = t;
    return;
  }
  const int W = windows_of(Kv);
  const float* sc = scores + (long long)b * cap;
  auto weight = [&](int w) -> uint32_t { return (uint32_t)min(kWin, Kv - kWin * w); };
  // thread t owns windows [t C, t C + C): consecutive in index order, so one
  // block scan orders them.  Staged, window t C + e sits at t (C + 1) + e: one pad
  // word per chunk keeps the chunk reads of a wave on distinct banks for even C,
  // and the reads of a chunk are one base address plus constant offsets.
  // w / C = (w ceil(2^31 / C)) >> 31 exactly for w < 2^15 and 1 <= C <= 32.
  const int C = (W + kSelThreads - 1) / kSelThreads;
  const int wbeg = min(W, tid * C), wend = min(W, wbeg + C);
  const uint32_t cmul = (0x80000000u + (unsigned)C - 1u) / (unsigned)C;   // fits: C >= 1
  auto slot = [cmul](int w) { return w + (int)(((uint64_t)(unsigned)w * cmul) >> 31); };

  // ---- scores -> LDS (every load in flight at once) and their min / max ----
  float lo = INFINITY, hi = -INFINITY;
  {
    constexpr int PER = kStage / kSelThreads;
    const int wst = min(W, kStage);
    float v[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int w = tid + kSelThreads * k;
      v[k] = w < wst ? sc[w] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int w = tid + kSelThreads * k;
      if (w < wst) {
        sk[slot(w)] = v[k];
        lo = fminf(lo, v[k]);
        hi = fmaxf(hi, v[k]);
      }
    }
    for (int w = kStage + tid; w < W; w += kSelThreads) {   // windows past the staged ones
      const float x = sc[w];
      lo = fminf(lo, x);
      hi = fmaxf(hi, x);
    }
  }
  // (the staged scores are read only after the barrier that publishes the min / max)
  // for_chunk(f) calls f(w, score of w) for this thread's windows in window order;
  // when every window is staged (the score array fits LDS), the LDS reads go in
  // batches of 8 independent loads; otherwise the scores come from memory.  (One
  // load whose address space depends on w would go through a generic pointer.)
  constexpr int PER = kStage / kSelThreads;
  constexpr int BATCH = 8;
  const bool staged = C <= PER;
  const int cbase = tid * (C + 1);   // LDS index of this thread's first window
  auto for_chunk = [&](auto f) __attribute__((always_inline)) {
    if (staged) {
#pragma unroll 1
      for (int e0 = 0; e0 < PER; e0 += BATCH) {   // rolled: the kernel's code stays small
        if (wbeg + e0 >= wend) break;
        float t[BATCH];
#pragma unroll
        for (int j = 0; j < BATCH; ++j) t[j] = sk[cbase + e0 + j];   // in bounds: tid (C + 1) + 31 < kStage + kStage / 32
#pragma unroll
        for (int j = 0; j < BATCH; ++j)
          if (wbeg + e0 + j < wend) f(wbeg + e0 + j, t[j]);
      }
    } else {   // more windows than LDS holds: read the scores from memory
      for (int w = wbeg; w < wend; ++w) f(w, sc[w]);
    }
  };
#pragma unroll
  for (int dd = 32; dd >= 1; dd >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, dd, kWave));
    hi = fmaxf(hi, __shfl_xor(hi, dd, kWave));
  }
  if (lane == 0) {
    mm[0][wv] = lo;
    mm[1][wv] = hi;
  }
  for (int k = tid; k < kBuckets; k += kSelThreads) bhist[k] = 0u;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kSelWaves; ++k) {
    lo = fminf(lo, mm[0][k]);
    hi = fmaxf(hi, mm[1][k]);
  }

  // ---- buckets: kBuckets equal slices of [min, max].  The bucket is a
  // non-decreasing function of the score (rounding is monotonic), so every
  // window of a higher bucket scores above every window of a lower one; only
  // the bucket holding the budget-th position needs the exact select.
  const float span = hi - lo;
  float scale = (span > 0.f && span < INFINITY) ? (float)kBuckets / span : 0.f;
  if (!(scale <= 3e38f)) scale = 0.f;   // a span too small to divide: one bucket
  auto bucket = [&](float x) -> int { return scale > 0.f ? min((int)((x - lo) * scale), kBuckets - 1) : 0; };
  for_chunk([&](int w, float x) __attribute__((always_inline)) { atomicAdd(&bhist[bucket(x)], weight(w)); });
  __syncthreads();
  uint32_t need = (uint32_t)budget;
  {
    // thread t: buckets j0 = kBuckets - 1 - 2t and j0 - 1; weight above j0 by a block scan
    static_assert(kBuckets == 2 * kSelThreads, "two buckets per thread");
    const int j0 = kBuckets - 1 - 2 * tid;
    const uint32_t h0 = bhist[j0], h1 = bhist[j0 - 1];
    uint64_t tot;
    const uint32_t above = (uint32_t)block_exscan_u64((uint64_t)(h0 + h1), scan_sh, &tot);
    if (above < need && need <= above + h0) {
      pick[0] = (uint32_t)j0;
      pick[1] = above;
    } else if (above + h0 < need && need <= above + h0 + h1) {
      pick[0] = (uint32_t)(j0 - 1);
      pick[1] = above + h0;
    }
    __syncthreads();
  }
  const int DB = (int)pick[0];
  need -= pick[1];
  __syncthreads();   // pick is written again by the radix select

  // ---- the windows of that bucket: a short list in LDS, unless there are too
  // many (then the select runs over every window, filtered by bucket)
  // tm: bit e marks window wbeg + e of a staged chunk when its bucket is DB or
  // above.  Bucket is monotone in the score, so every window the selection takes
  // is marked, and the count and the placement visit only the marked ones.
  uint32_t tm = 0u;
  for_chunk([&](int w, float x) __attribute__((always_inline)) {
    const int bk = bucket(x);
    if (bk == DB) {
      const uint32_t c = atomicAdd(&ncand, 1u);
      if (c < kCand) {
        cand[c][0] = order_key(x);
        cand[c][1] = weight(w);
      }
    }
    tm |= (bk >= DB ? 1u : 0u) << ((w - wbeg) & 31);   // used only when staged (C <= 32)
  });
  __syncthreads();
  const uint32_t nc = ncand;
  uint32_t ukey;
  if (nc <= kCand) {
    if (wv == 0) {
      const uint32_t k = nc <= (uint32_t)kWave ? wave_rank_list(cand, nc, &need)
                                               : wave_radix_list(cand, nc, &need, &hist[0][0]);
      if (lane == 0) {
        pick[0] = k;
        pick[1] = need;
      }
    }
    __syncthreads();
    ukey = pick[0];
    need = pick[1];
  } else {
    ukey = radix_select([&](auto f) __attribute__((always_inline)) {
      for_chunk([&](int w, float x) __attribute__((always_inline)) {
        if (bucket(x) == DB) f(order_key(x), weight(w));
      });
    }, &need, hist, pick);
  }
  // ukey = key of the last window taken; `need` positions come from the
  // windows of exactly that key, in window order.

  // ---- placement: this thread's windows, after every earlier thread's ----------
  // for_taken(f): f(w, score) for the windows that can be taken, in window order
  // (the rest add nothing to either count)
  auto for_taken = [&](auto f) __attribute__((always_inline)) {
    if (staged) {
      for (uint32_t m = tm; m != 0u; m &= m - 1u) {
        const int e = __builtin_ctz(m);
        f(wbeg + e, sk[cbase + e]);
      }
    } else {
      for_chunk(f);
    }
  };
  uint32_t sg = 0u, se = 0u;
  for_taken([&](int w, float x) __attribute__((always_inline)) {
    const uint32_t u = order_key(x), c = weight(w);
    sg += u > ukey ? c : 0u;   // branch-free: the two counters stay in registers
    se += u == ukey ? c : 0u;
  });
  uint64_t tot;
  const uint64_t ex = block_exscan_u64(((uint64_t)se << 32) | sg, scan_sh, &tot);
  uint32_t gb = (uint32_t)ex, eb = (uint32_t)(ex >> 32);
  if (sg + se > 0u) {
    for_taken([&](int w, float x) __attribute__((always_inline)) {
      const uint32_t u = order_key(x);
      const uint32_t c = weight(w);
      // positions taken before window w: all of the higher windows, and the
      // tied windows in order until `need` is met
      const uint32_t pos = gb + min(eb, need);
      const uint32_t n = u > ukey ? c : (u == ukey ? min(c, need - min(eb, need)) : 0u);
      if (n > 0u) {   // skipped by the whole wave when none of its lanes takes this window
#pragma unroll
        for (uint32_t j = 0; j < (uint32_t)kWin; ++j) {
          const uint32_t p = pos + j;
          if (j < n && p < (uint32_t)budget) {
            if (p < (uint32_t)kOutStage)
              aux[p] = (uint32_t)(kWin * w) + j;   // written out in order below
            else
              out[p] = kWin * w + (int)j;
          }
        }
      }
      gb += u > ukey ? c : 0u;
      eb += u == ukey ? c : 0u;
    });
  }
  __syncthreads();
  const int nstage = min(budget, kOutStage);
  for (int p = tid; p < nstage; p += kSelThreads) out[p] = (int32_t)aux[p];
}

// ---- launchers ------------------------------------------------------------------
hipError_t indexer_pool(const void* keys, long long ld, const int32_t* off_dev, int B, int d, int S, bool full,
                        int wmax, float* pooled, int cap, hipStream_t st) {
  if (wmax <= 0) return hipSuccess;
  hipLaunchKernelGGL(pool_windows_kernel, dim3((wmax + 3) / 4, B), dim3(256), 0, st, (const uint16_t*)keys, ld,
                     off_dev, d, S, full ? 1 : 0, pooled, cap);
  return hipGetLastError();
}

hipError_t indexer_pool_fixed(const void* keys, long long ld, const int32_t* off_dev, int B, int d, int S, int P,
                              float* pooled, int cap, hipStream_t st) {
  hipLaunchKernelGGL(pool_fixed_kernel, dim3(P / 4, B), dim3(256), 0, st, (const uint16_t*)keys, ld, off_dev, d, S,
                     pooled, cap);
  return hipGetLastError();
}

hipError_t indexer_scores(float* pooled, int cap, int d, const float* q, const int32_t* off_dev, int B, int wmax,
                          float* scores, const uint16_t* tail_keys, long long tail_ld, int tail_S, hipStream_t st) {
  const int per_block = 4 * kScoreWin;
  const int gx = std::min((wmax + per_block - 1) / per_block, std::max(1, kScoreBlocks / B));
  const TailArgs ta{tail_keys, tail_ld, tail_S};
  const dim3 grid(gx + (tail_keys ? 1 : 0), B);   // + the workgroup that pools and scores the tail
  if (tail_keys) {
    if (d <= 2 * 4 * kWave)
      hipLaunchKernelGGL((window_scores_kernel<2, true>), grid, dim3(256), 0, st, pooled, cap, d, q, off_dev, scores, ta);
    else
      hipLaunchKernelGGL((window_scores_kernel<4, true>), grid, dim3(256), 0, st, pooled, cap, d, q, off_dev, scores, ta);
  } else {
    if (d <= 2 * 4 * kWave)
      hipLaunchKernelGGL((window_scores_kernel<2, false>), grid, dim3(256), 0, st, pooled, cap, d, q, off_dev, scores, ta);
    else
      hipLaunchKernelGGL((window_scores_kernel<4, false>), grid, dim3(256), 0, st, pooled, cap, d, q, off_dev, scores, ta);
  }
  return hipGetLastError();
}

hipError_t indexer_select(const float* scores, int cap, const int32_t* off_dev, int B, int budget,
                          const int32_t* sel_off_dev, int32_t* sel, hipStream_t st) {
  hipLaunchKernelGGL(select_positions_kernel, dim3(B), dim3(kSelThreads), 0, st, scores, cap, off_dev, budget,
                     sel_off_dev, sel);
  return hipGetLastError();
}

}  // namespace mla
