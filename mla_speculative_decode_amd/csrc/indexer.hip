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
// budget-th position, a weighted radix select (8-bit digits of the score's
// order key, weight = positions in the window) inside that slice finds the
// score of the last window taken, and a scan over windows in index order then
// places each taken window's positions.  Integer work only after the scores: the selection
// of given scores is exact.

#include "mla_device.h"
#include "internal.h"

namespace mla {

constexpr int kWin = 4;

__device__ __forceinline__ int windows_of(int T) { return (T + kWin - 1) / kWin; }

// ---- pooling ----------------------------------------------------------------
// grid (ceil(wmax / 4), B), 256 threads: one wave per window, lane l takes the
// 8-column chunks l, l + 64, ...
__global__ __launch_bounds__(256) void pool_windows_kernel(const uint16_t* __restrict__ keys, long long ld,
                                                           const int32_t* __restrict__ off, int d, int S, int full,
                                                           float* __restrict__ pooled, int cap) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.y;
  const int o0 = off[b];
  const int Kv = off[b + 1] - o0;
  const int first = full ? 0 : (Kv - S) / kWin;
  const int w = first + blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= windows_of(Kv)) return;
  const int n = min(kWin, Kv - kWin * w);
  const uint16_t* src = keys + ((long long)o0 + kWin * w) * ld;
  float* dst = pooled + ((long long)b * cap + w) * d;
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

// ---- scores -----------------------------------------------------------------
// grid (ceil(wmax / 16), B), 256 threads: wave v takes windows 16 x + 4 v ..
// + 3, lane l the float4 chunks l, l + 64, ... (d <= 1024: at most 4).
constexpr int kScoreWin = 4;   // windows per wave
__global__ __launch_bounds__(256) void window_scores_kernel(const float* __restrict__ pooled, int cap, int d,
                                                            const float* __restrict__ q,
                                                            const int32_t* __restrict__ off,
                                                            float* __restrict__ scores) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.y;
  const int W = windows_of(off[b + 1] - off[b]);
  const int w0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * kScoreWin;
  if (w0 >= W) return;
  const int nc = d / 4;
  f32x4 qv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = lane + kWave * j;
    qv[j] = c < nc ? *reinterpret_cast<const f32x4*>(q + (long long)b * d + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  f32x4 pv[kScoreWin][4];
#pragma unroll
  for (int k = 0; k < kScoreWin; ++k) {
    const int w = min(w0 + k, W - 1);
    const float* row = pooled + ((long long)b * cap + w) * d;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = lane + kWave * j;
      pv[k][j] = c < nc ? *reinterpret_cast<const f32x4*>(row + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
#pragma unroll
  for (int k = 0; k < kScoreWin; ++k) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) s = fmaf(qv[j][e], pv[k][j][e], s);
#pragma unroll
    for (int dd = 32; dd >= 1; dd >>= 1) s += __shfl_xor(s, dd, kWave);
    if (lane == 0 && w0 + k < W) scores[(long long)b * cap + w0 + k] = s;
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
__device__ uint32_t radix_select(ForEach for_each, uint32_t* need, uint32_t (*hist)[256], uint32_t* pick) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  uint32_t prefix = 0u, mask = 0u;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int k = tid; k < kHistCopies * 256; k += kSelThreads) (&hist[0][0])[k] = 0u;
    __syncthreads();
    for_each([&](uint32_t u, uint32_t wgt) {
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

// grid B, 1024 threads: one block per sequence.
__global__ __launch_bounds__(kSelThreads) void select_positions_kernel(const float* __restrict__ scores, int cap,
                                                                       const int32_t* __restrict__ off, int budget,
                                                                       const int32_t* __restrict__ sel_off,
                                                                       int32_t* __restrict__ sel) {
  __shared__ uint32_t hist[kHistCopies][256];
  __shared__ uint32_t bhist[kBuckets];
  __shared__ float sk[kStage + kStage / 32];   // the first kStage window scores (a pad word every 32)
  __shared__ uint32_t cand[kCand][2];   // (order key, weight) of the windows in the boundary bucket
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
  // block scan orders them; the pad word makes the chunk reads conflict-free
  const int C = (W + kSelThreads - 1) / kSelThreads;
  const int wbeg = min(W, tid * C), wend = min(W, wbeg + C);
  auto slot = [](int w) { return w + (w >> 5); };

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
  auto val = [&](int w) -> float { return w < kStage ? sk[slot(w)] : sc[w]; };
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
  for (int w = wbeg; w < wend; ++w) atomicAdd(&bhist[bucket(val(w))], weight(w));
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
  for (int w = wbeg; w < wend; ++w) {
    const float x = val(w);
    if (bucket(x) == DB) {
      const uint32_t c = atomicAdd(&ncand, 1u);
      if (c < kCand) {
        cand[c][0] = order_key(x);
        cand[c][1] = weight(w);
      }
    }
  }
  __syncthreads();
  const uint32_t nc = ncand;
  uint32_t ukey;
  if (nc <= kCand) {
    ukey = radix_select([&](auto f) {
      for (uint32_t c = tid; c < nc; c += kSelThreads) f(cand[c][0], cand[c][1]);
    }, &need, hist, pick);
  } else {
    ukey = radix_select([&](auto f) {
      for (int w = wbeg; w < wend; ++w) {
        const float x = val(w);
        if (bucket(x) == DB) f(order_key(x), weight(w));
      }
    }, &need, hist, pick);
  }
  // ukey = key of the last window taken; `need` positions come from the
  // windows of exactly that key, in window order.

  // ---- placement: this thread's windows, after every earlier thread's ----------
  uint32_t sg = 0u, se = 0u;
  for (int w = wbeg; w < wend; ++w) {
    const uint32_t u = order_key(val(w));
    if (u > ukey) sg += weight(w);
    else if (u == ukey) se += weight(w);
  }
  uint64_t tot;
  const uint64_t ex = block_exscan_u64(((uint64_t)se << 32) | sg, scan_sh, &tot);
  uint32_t gb = (uint32_t)ex, eb = (uint32_t)(ex >> 32);
  if (sg + se > 0u) {
    for (int w = wbeg; w < wend; ++w) {
      const uint32_t u = order_key(val(w));
      const uint32_t c = weight(w);
      // positions taken before window w: all of the higher windows, and the
      // tied windows in order until `need` is met
      const uint32_t pos = gb + min(eb, need);
      const uint32_t n = u > ukey ? c : (u == ukey ? min(c, need - min(eb, need)) : 0u);
      for (uint32_t j = 0; j < n && pos + j < (uint32_t)budget; ++j) out[pos + j] = kWin * w + (int)j;
      if (u > ukey) gb += c;
      else if (u == ukey) eb += c;
    }
  }
}

// ---- launchers ------------------------------------------------------------------
hipError_t indexer_pool(const void* keys, long long ld, const int32_t* off_dev, int B, int d, int S, bool full,
                        int wmax, float* pooled, int cap, hipStream_t st) {
  if (wmax <= 0) return hipSuccess;
  hipLaunchKernelGGL(pool_windows_kernel, dim3((wmax + 3) / 4, B), dim3(256), 0, st, (const uint16_t*)keys, ld,
                     off_dev, d, S, full ? 1 : 0, pooled, cap);
  return hipGetLastError();
}

hipError_t indexer_scores(const float* pooled, int cap, int d, const float* q, const int32_t* off_dev, int B,
                          int wmax, float* scores, hipStream_t st) {
  const int per_block = 4 * kScoreWin;
  hipLaunchKernelGGL(window_scores_kernel, dim3((wmax + per_block - 1) / per_block, B), dim3(256), 0, st, pooled,
                     cap, d, q, off_dev, scores);
  return hipGetLastError();
}

hipError_t indexer_select(const float* scores, int cap, const int32_t* off_dev, int B, int budget,
                          const int32_t* sel_off_dev, int32_t* sel, hipStream_t st) {
  hipLaunchKernelGGL(select_positions_kernel, dim3(B), dim3(kSelThreads), 0, st, scores, cap, off_dev, budget,
                     sel_off_dev, sel);
  return hipGetLastError();
}

}  // namespace mla
