// split_absorbed.hip -- the split-KV kernel of the absorbed MLA route over a
// bf16 latent cache (pages: "One guard, 110x off the verify step", section
// "The defect": attend directly against the compressed latent and accumulate
// in latent space).
//
// The absorbed route is multi-query attention with one shared key/value head:
// every (row, head) pair of a sequence is a query of width 512 + rope against
// the keys [c_kv | k_pe], and the values are c_kv itself.  A workgroup takes 64
// query rows x one split of the sequence's positions, in tiles of 64 positions
// held in LDS, and leaves unnormalised partial results (latent sums in bf16, the
// row's base-2 reference and sum in float32) for the merge pass.
//
// Layout of the four waves:
//   scores  wave w computes S^T for keys 16w .. 16w+15 of the tile against all
//           64 query rows with 16x16x32 bf16 MFMAs: the query block of all 64
//           rows stays in registers (B operand), and each key fragment read from
//           LDS feeds four MFMAs (one per block of 16 rows);
//   softmax base 2 against a fixed reference per row (the row's maximum over the
//           split's first tile); a lane holds 4 keys of 4 rows, so P, the row
//           sums and the running maxima need no exchange between lanes inside
//           the tile loop; a split whose later scores exceed the reference by
//           more than 2^64 runs again with the references raised;
//   PV      O^T[512 x 64 rows] += V^T P^T with 32x32x16 MFMAs, wave w owning
//           latent columns 128w .. 128w+127; P (bf16) comes from LDS, V^T
//           fragments are read transposed from the row-major tile with
//           ds_read_b64_tr_b16.
// LDS: two latent tile buffers (the tile being scored and the next one, copied
// in by direct global -> LDS loads spread over the score MFMAs, one 1 KB latent
// row per wave instruction), one rope-key buffer (the next tile's rope keys are
// copied in during PV, after every wave has scored the current ones), the rope
// part of the query block (its latent part lives in registers), and P with
// the per-row exchange slots in its pad column.  The selected-position form
// (SEL) runs over a per-sequence list of cache positions instead of all of
// them.

#include <algorithm>
#include <type_traits>

#include "mla_device.h"
#include "internal.h"

namespace mla {

namespace {

struct SplitArgs {
  const uint16_t* q_lat;   // [B, L, H, 512]
  const uint16_t* q_pe;    // [B, L, H, DR]
  const uint16_t* c_kv;    // [T, 512]
  const uint16_t* k_pe;    // [T, DR]
  const int32_t* sel;      // SEL: selected positions per sequence (packed by off; relative, increasing)
  const int32_t* koff;     // SEL: cache offsets [B+1] (off then indexes the selection)
  int koff0, kvt1;         // SEL, B == 1: koff[0] and koff[1] - koff[0]
  const int32_t* off;      // [B+1] device offsets
  int off0, kv1;           // B == 1: off[0] and off[1] - off[0]
  uint16_t* ws_o;          // [G][rows][512] unnormalised partial sums, bf16
  float* ws_ml;            // [G][rows][2]: base-2 reference, row sum
  int B, L, H;
  int rows;                // L * H query rows per sequence
  int row_tiles;           // ceil(rows / 64)
  int pf_ahead;            // tiles of L2 prefetch ahead of the tile being scored
  int chunk;               // positions per split (multiple of 64)
  int n_items;
  float sl2;               // scale * log2(e)
};

constexpr float kRefSlack = 64.f;   // P = 2^(s - m) <= 2^64 keeps bf16 / float32 exact in relative terms

// Reductions over the four 16-lane groups (lanes l, l^16, l^32, l^48 hold the
// same row) with gfx950's lane swaps: after a 32-lane and a 16-lane swap of
// x with itself, the two halves of each pair hold the values of the lanes
// 32 apart, then 16 apart.
__device__ __forceinline__ float group_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace

template <int DR, bool SEL>
__global__ __launch_bounds__(256, 1) void absorbed_split_kernel(SplitArgs p) {
  constexpr int DA = 512, DV = 512;
  constexpr int BM = 64, BN = 64;
  constexpr int KL = DA / 32;             // 32-wide k steps of the score MFMA over the latent part
  constexpr int KR = DR / 32;             // ... over the rope part
  // Latent LDS row: 1 KB + 48 B of pad, a stride of 48 mod 256 bytes: the 16
  // rows a score fragment reads fall in 16 distinct bank groups, and the rows
  // of a transposed V read in 4 distinct 64-byte windows.
  constexpr int LRB = DA * 2 + 48;
  constexpr int RCH = DR / 8;             // 16-byte rope chunks per row (8 at rope 64)
  constexpr int RRB = RCH * 16;           // rope LDS row: unpadded, chunk c of row r stored at c ^ (r & 7)
  constexpr int RINST = BN * RCH / kWave; // rope direct-load wave instructions per tile (8 rows each)
  constexpr int BUF = BN * LRB;
  constexpr int RBUF = DR > 0 ? BN * RRB : 16;
  constexpr int PRB = 9 * 16;             // P row: 64 keys (8 chunks) + one chunk holding 4 exchange floats
  constexpr int CPW = DV / 4;             // value columns per wave
  constexpr int NCB = CPW / 32;           // 32-column MFMA blocks per wave
  constexpr int NLW = BN / 4;             // latent-row copy instructions per wave per tile
  static_assert(DR % 32 == 0 && (DR == 0 || RCH == 8), "rope width 0 or 64");

  __shared__ __attribute__((aligned(1024))) uint8_t buf0[BUF];
  __shared__ __attribute__((aligned(1024))) uint8_t buf1[BUF];
  __shared__ __attribute__((aligned(16))) uint8_t krope[RBUF];   // rope keys of the tile being scored
  __shared__ __attribute__((aligned(16))) uint8_t qrope[RBUF];   // rope part of the query block
  __shared__ __attribute__((aligned(16))) uint8_t pl[BM * PRB];
  __shared__ uint32_t pfd[kWave];   // landing slot of the L2 prefetch (never read)
  // per-row exchange slots: row r's four floats (one per wave) in P's pad chunk
  auto red = [&](int row) -> float* { return reinterpret_cast<float*>(pl + row * PRB + 128); };

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;          // score layout: row block lane, key group
  const int half = lane >> 5, l32 = lane & 31;        // PV layout
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int item = __builtin_amdgcn_readfirstlane(xcd_item(blockIdx.x, p.n_items));
  if (item >= p.n_items) return;
  const int rt = __builtin_amdgcn_readfirstlane(item % p.row_tiles);
  const int g = __builtin_amdgcn_readfirstlane(item / p.row_tiles);
  int b = 0, ps = g, off_b = p.off0, Kv = p.kv1;
  if (p.B > 1) {
    const SplitPos sp = decode_split(g, p.off, p.B, p.chunk);
    b = __builtin_amdgcn_readfirstlane(sp.b);
    ps = __builtin_amdgcn_readfirstlane(sp.s);
    off_b = __builtin_amdgcn_readfirstlane(p.off[b]);
    Kv = __builtin_amdgcn_readfirstlane(p.off[b + 1]) - off_b;
  }
  // SEL: off_b / Kv index the packed selection; cache rows start at koff[b] and
  // the causal bound comes from the cache length Kt.
  long long p0 = off_b;
  int Kt = Kv;
  if (SEL) {
    p0 = p.B > 1 ? (long long)__builtin_amdgcn_readfirstlane(p.koff[b]) : (long long)p.koff0;
    Kt = p.B > 1 ? __builtin_amdgcn_readfirstlane(p.koff[b + 1]) - (int)p0 : p.kvt1;
  }
  const int sel0 = off_b;
  const int k0 = __builtin_amdgcn_readfirstlane(ps * p.chunk);
  const int k1 = __builtin_amdgcn_readfirstlane(min(Kv, k0 + p.chunk));
  // SEL: entries at or above a row's bound Kt - L + i + 1 are among the
  // selection's last L - 1; lane j holds the j-th entry from the end.
  const int ntail = min(p.L - 1, Kv);
  int tailv = -1;
  if (SEL && ntail <= kWave && lane < ntail) tailv = p.sel[sel0 + Kv - 1 - lane];
  auto visible = [&](int i) -> int {   // split indices query row i may see
    const int bound = Kt - p.L + i + 1;
    if (!SEL) return bound;
    if (ntail <= kWave) {
      int above = 0;
      for (int j = 0; j < ntail; ++j) above += __builtin_amdgcn_readlane(tailv, j) >= bound ? 1 : 0;
      return Kv - above;
    }
    int lo = 0, hi = Kv;               // long blocks: binary search of the increasing selection
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (p.sel[sel0 + mid] < bound) lo = mid + 1; else hi = mid;
    }
    return lo;
  };
  // SEL: cache positions of the 64 keys of the next tile to copy (lane j: key j)
  int sidx = 0;
  auto load_idx = [&](int t0) {
    if (SEL) sidx = min(max(p.sel[sel0 + min(t0 + lane, k1 - 1)], 0), Kt - 1);
  };
  const int idx0 = rt * BM;
  const int nrows = min(BM, p.rows - idx0);

  const uint16_t* lbase = uniform_ptr(p.c_kv + p0 * DA);
  const uint16_t* rseq = p.k_pe + p0 * DR;

  // ---- tile copy: global -> LDS --------------------------------------------
  // latent row `key` of the tile: one wave instruction (uniform row address,
  // lane l copies bytes 16 l .. 16 l + 15)
  auto issue_part = [&](int t0, uint8_t* kdst, int x) {
    const int key = wu + 4 * x;
    const int kr = SEL ? __builtin_amdgcn_readlane(sidx, key) : __builtin_amdgcn_readfirstlane(min(t0 + key, k1 - 1));
    __builtin_amdgcn_global_load_lds(lbase + (long long)kr * DA + 8 * lane,
                                     (__attribute__((address_space(3))) void*)(kdst + key * LRB), 16, 0, 0);
  };
  // rope keys of the tile into krope: instruction j fills rows 8 j .. 8 j + 7;
  // lane l lands in row 8 j + l / 8, physical chunk l % 8, so it loads logical
  // chunk (l % 8) ^ (l / 8) of that row
  const int rsw = (lane & 7) ^ (lane >> 3);
  auto issue_rope = [&](int t0) {
#pragma unroll
    for (int x = 0; x < RINST / 4; ++x) {
      const int j = wu + 4 * x;
      const int key = 8 * j + (lane >> 3);
      const int kr = SEL ? __shfl(sidx, key, kWave) : min(t0 + key, k1 - 1);
      __builtin_amdgcn_global_load_lds(rseq + (long long)kr * DR + 8 * rsw,
                                       (__attribute__((address_space(3))) void*)(krope + 1024 * j), 16, 0, 0);
    }
  };
  auto issue_tile = [&](int t0, uint8_t* kdst) {
    if (DR > 0) issue_rope(t0);
#pragma unroll
    for (int x = 0; x < NLW; ++x) issue_part(t0, kdst, x);
  };

  // ---- rows of this lane in the score layout: 16 rb + l16, rb < 4 ----------
  int kend[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int idx = idx0 + min(16 * rb + l16, nrows - 1);
    kend[rb] = min(k1, visible(idx / p.H));
  }
  const int kfull = __builtin_amdgcn_readfirstlane(min(k1, visible(idx0 / p.H)));   // every row sees these

  load_idx(k0);
  issue_tile(k0, buf0);   // first tile in flight while the queries load
  load_idx(k0 + BN);

  // ---- query block: latent part -> buf1 -> registers; rope part -> qrope -----
  // Rows past the last query row repeat it (their results are never stored).
  u32x4 qf[4][KL];
  {
    const long long qflat0 = (long long)b * p.rows + idx0;
    const uint16_t* qlseq = p.q_lat + qflat0 * DA + 8 * lane;
#pragma unroll
    for (int x = 0; x < BM / 4; ++x) {
      const int row = wu + 4 * x;
      __builtin_amdgcn_global_load_lds(qlseq + (long long)min(row, nrows - 1) * DA,
                                       (__attribute__((address_space(3))) void*)(buf1 + row * LRB), 16, 0, 0);
    }
    if (DR > 0) {   // same swizzled layout as the rope keys
#pragma unroll
      for (int x = 0; x < RINST / 4; ++x) {
        const int j = wu + 4 * x;
        const int row = 8 * j + (lane >> 3);
        __builtin_amdgcn_global_load_lds(p.q_pe + (qflat0 + min(row, nrows - 1)) * DR + 8 * rsw,
                                         (__attribute__((address_space(3))) void*)(qrope + 1024 * j), 16, 0, 0);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // the query fragments are read from buf1 by the first tile's score loop
    // (each as its MFMAs need it); tile 1 is copied into buf1 after that
  }

  // ---- running state (score layout: row 16 rb + l16) -----------------------
  float m_ref[4], l_part[4], t_max[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) { m_ref[rb] = -INFINITY; l_part[rb] = 0.f; t_max[rb] = -INFINITY; }
  bool rerun = false;
  f32x16 O[2][NCB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) O[rb][cb][i] = 0.f;

  // per-lane LDS offsets (bytes) within a buffer; the rest are immediates
  const int kq_off = (16 * w + l16) * LRB + 16 * lg;                     // + 64 ks
  // rope rows (row & 7 == l16 & 7 in both): chunk c at (c ^ (l16 & 7)), c = 4 ks + lg
  auto rope_off = [&](int ks) { return 16 * ((4 * ks + lg) ^ (l16 & 7)); };
  const int kr_off = (16 * w + l16) * RRB;                               // rope keys
  const int qr_off = l16 * RRB;                                          // rope queries: + 16 rb RRB
  const int G = lane >> 4, s16 = lane & 15;
  const int tr_off = (8 * (G >> 1) + (s16 >> 2)) * LRB + (w * CPW + 16 * (G & 1) + 4 * (s16 & 3)) * 2;
  const int pa_off = l32 * PRB + 16 * half;                              // + rb*32*PRB + 32 kc
  const int pw_off = l16 * PRB + (16 * w + 4 * lg) * 2;                  // + 16 rb * PRB

  // Cache lines of the split's positions [ta, tb) -> L2 ahead of their tile
  // copies: this workgroup takes the positions p with (p - k0) % row_tiles == rt,
  // one 4-byte load per 128-byte line into a dummy LDS slot (the row tiles of a
  // split run on one XCD and share its L2).  Each tile fetches the lines of the
  // tile pf_ahead tiles on; the first one fetches the tiles up to there.
  const int kPfAhead = p.pf_ahead;
  auto prefetch_range = [&](int ta, int tb) {
    if (SEL) return;
    constexpr int LPP = DA / 64 + (DR > 0 ? 1 : 0);   // 128-byte lines per position
    tb = min(tb, k1);
    const int rel = ta - k0;
    const int first = ta + ((rt - rel % p.row_tiles) + p.row_tiles) % p.row_tiles;
    const int cnt = first < tb ? (tb - 1 - first) / p.row_tiles + 1 : 0;
    const int nl = cnt * LPP;
    for (int e0 = 0; e0 < nl; e0 += 256) {
      const int e = min(e0 + tid, nl - 1);
      const int j = e / LPP, ln = e - j * LPP;
      const long long pos = p0 + first + (long long)p.row_tiles * j;
      const uint16_t* src = ln < DA / 64 ? p.c_kv + pos * DA + 64 * ln : p.k_pe + pos * DR;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)pfd, 4, 0, 0);
    }
  };

  // Scores of one tile over the latent part.  LQ: the first tile, whose query
  // fragments are read from buf1 as the MFMAs need them (two k steps ahead).
  // NC: how many of the next tile's 16 latent-row copies to issue here (the
  // rest go with PV, so that neither phase carries all of the copy's LDS writes).
  auto latent_scores = [&](f32x4* acc, const uint8_t* cur, uint8_t* nxt, int t1, auto lq, auto nc) {
    constexpr bool LQ = decltype(lq)::value;
    constexpr int NC = decltype(nc)::value;
    constexpr int PF = 4, QPF = 2;
    const uint8_t* kq = cur + kq_off;
    const uint8_t* qsrc = buf1 + l16 * LRB + 16 * lg;
    u32x4 ka[PF];
    if (LQ) {
#pragma unroll
      for (int ks = 0; ks < QPF; ++ks)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) qf[rb][ks] = *reinterpret_cast<const u32x4*>(qsrc + 16 * rb * LRB + 64 * ks);
    }
#pragma unroll
    for (int c = 0; c < PF; ++c) ka[c] = *reinterpret_cast<const u32x4*>(kq + 64 * c);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < KL; ++ks) {
      const u32x4 a = ka[ks % PF];
      if (ks + PF < KL) ka[ks % PF] = *reinterpret_cast<const u32x4*>(kq + 64 * (ks + PF));
      if (LQ && ks + QPF < KL) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
          qf[rb][ks + QPF] = *reinterpret_cast<const u32x4*>(qsrc + 16 * rb * LRB + 64 * (ks + QPF));
      }
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) acc[rb] = mfma16(a, qf[rb][ks], acc[rb]);
      if (NC > 0) {
#pragma unroll
        for (int x = (ks * NC) / KL; x < ((ks + 1) * NC) / KL; ++x) issue_part(t1, nxt, x);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // one 64-position tile: scores from `cur`, copy of the next tile into `nxt`
  auto step = [&](int t0, const uint8_t* cur, uint8_t* nxt, bool pf) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // (A) tile t visible; PV(t-1) done, so the other buffer and pl are free
    // the split's first tile on the first pass: the query fragments come from
    // buf1 during its scores, so the next tile's copy waits for PV
    const bool first = t0 == k0 && !rerun;
    if (!rerun) {
      if (first) prefetch_range(t0 + BN, t0 + (kPfAhead + 1) * BN);
      else prefetch_range(t0 + kPfAhead * BN, t0 + (kPfAhead + 1) * BN);
    }

    // ---- scores: S^T [16 keys x 64 rows] -----------------------------------
    f32x4 acc[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // rope part first, from LDS on both sides (its registers are free again for the latent part)
#pragma unroll
    for (int ks = 0; ks < KR; ++ks) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(krope + kr_off + rope_off(ks));
      u32x4 bq[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) bq[rb] = *reinterpret_cast<const u32x4*>(qrope + qr_off + 16 * rb * RRB + rope_off(ks));
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) acc[rb] = mfma16(a, bq[rb], acc[rb]);
    }
    using I0 = std::integral_constant<int, 0>;
    using IH = std::integral_constant<int, NLW / 2>;
    if (first) latent_scores(acc, cur, nxt, t0 + BN, std::true_type{}, I0{});
    else if (pf) latent_scores(acc, cur, nxt, t0 + BN, std::false_type{}, IH{});
    else latent_scores(acc, cur, nxt, t0 + BN, std::false_type{}, I0{});
    // latent-row copies of the next tile still to issue (during PV): x0 .. NLW - 1
    const int x0 = first ? 0 : NLW / 2;
    // acc[rb][i] = q . k for key t0 + 16 w + 4 lg + i, row 16 rb + l16.
    if (t0 + BN > kfull) {   // a tile past some row's causal end (uniform branch)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (t0 + 16 * w + 4 * lg + i >= kend[rb]) acc[rb][i] = -INFINITY;
    }
    // raw maxima (scaled once at the end: the scale is positive)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
      t_max[rb] = fmaxf(fmaxf(t_max[rb], fmaxf(acc[rb][0], acc[rb][1])), fmaxf(acc[rb][2], acc[rb][3]));
    // The first tile of the split sets each row's reference (a row sees a prefix
    // of the split's positions, so its first finite scores are in this tile).
    if (t0 == k0 && !rerun) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const float mx = group_max(fmaxf(fmaxf(acc[rb][0], acc[rb][1]), fmaxf(acc[rb][2], acc[rb][3])));
        if (lg == 0) red(16 * rb + l16)[w] = mx * p.sl2;
      }
      lds_barrier();
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const f32x4 r4 = *reinterpret_cast<const f32x4*>(red(16 * rb + l16));
        m_ref[rb] = fmaxf(fmaxf(r4[0], r4[1]), fmaxf(r4[2], r4[3]));
      }
    }
    // P = 2^(s - m) in bf16 (rows without a finite reference use 0: their masked
    // keys give 0); the row sums add the rounded weights that PV uses
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const float mb = m_ref[rb] == -INFINITY ? 0.f : m_ref[rb];
      float e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) e[i] = __builtin_amdgcn_exp2f(fmaf(acc[rb][i], p.sl2, -mb));
      u32x2 v;
      v[0] = pack_bf16(e[0], e[1]);
      v[1] = pack_bf16(e[2], e[3]);
      *reinterpret_cast<u32x2*>(pl + pw_off + 16 * rb * PRB) = v;
      l_part[rb] = add_bf16x2(v[1], add_bf16x2(v[0], l_part[rb]));
    }
    lds_barrier();  // (B) P visible (the next tile's copy stays in flight)
    // every wave has scored this tile's rope keys: copy the next tile's in
    if (DR > 0 && pf) issue_rope(t0 + BN);

    // ---- PV: O^T [CPW columns x 64 rows] for this wave's columns --------------
    {
      const uint8_t* pa = pl + pa_off;
      const uint8_t* vb = cur + tr_off;
      auto vfrag = [&](int kc, int cb) {
        u32x4 bv;
#pragma unroll
        for (int ld = 0; ld < 2; ++ld) {
          const uint8_t* src = vb + (16 * kc + 4 * ld) * LRB + 64 * cb;
          const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(src));
          const u32x2 rr = __builtin_bit_cast(u32x2, r);
          bv[2 * ld] = rr[0];
          bv[2 * ld + 1] = rr[1];
        }
        return bv;
      };
      constexpr int NSTEP = (BN / 16) * NCB;
      constexpr int VPF = 3;
      u32x4 a[BN / 16][2];
      u32x4 vq[VPF];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) a[0][rb] = *reinterpret_cast<const u32x4*>(pa + rb * 32 * PRB);
#pragma unroll
      for (int st = 0; st < VPF; ++st) {
        if (st > 0 && st % NCB == 0) {
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            a[st / NCB][rb] = *reinterpret_cast<const u32x4*>(pa + rb * 32 * PRB + 32 * (st / NCB));
        }
        vq[st] = vfrag(st / NCB, st % NCB);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int st = 0; st < NSTEP; ++st) {
        const int kc = st / NCB, cb = st % NCB;
        const u32x4 bcur = vq[st % VPF];
        const int sn = st + VPF;
        if (sn < NSTEP) {
          if (sn % NCB == 0) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
              a[sn / NCB][rb] = *reinterpret_cast<const u32x4*>(pa + rb * 32 * PRB + 32 * (sn / NCB));
          }
          vq[st % VPF] = vfrag(sn / NCB, sn % NCB);
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) O[rb][cb] = mfma32(bcur, a[kc][rb], O[rb][cb]);   // O^T += V^T P^T
        // this PV step's share of the next tile's remaining latent-row copies
        // (copy x at PV step x; the first tile's at every step, later ones' at steps 8 ..)
        if (pf && st >= x0) issue_part(t0 + BN, nxt, st);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    load_idx(t0 + 2 * BN);
  };

  for (;;) {
    for (int t0 = k0; t0 < k1; t0 += 2 * BN) {
      step(t0, buf0, buf1, t0 + BN < k1);
      if (t0 + BN < k1) step(t0 + BN, buf1, buf0, t0 + 2 * BN < k1);
    }
    // Did some row's scores exceed its reference by more than 2^kRefSlack?  Then
    // its P, O and l may have overflowed: raise every reference to the row's
    // maximum over the whole split and run the split again (the second pass
    // cannot trigger another: its references bound every score).
    __syncthreads();   // every wave is done with red and the tile buffers
    float tm[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const float mx = group_max(t_max[rb]);
      if (lg == 0) red(16 * rb + l16)[w] = mx * p.sl2;
    }
    lds_barrier();
    bool over = false;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const f32x4 r4 = *reinterpret_cast<const f32x4*>(red(16 * rb + l16));
      tm[rb] = fmaxf(fmaxf(r4[0], r4[1]), fmaxf(r4[2], r4[3]));
      over = over || (m_ref[rb] != -INFINITY && tm[rb] > m_ref[rb] + kRefSlack);
    }
    // every wave holds all 64 rows, so the decision is uniform over the
    // workgroup; the second pass never runs a third (its references bound every
    // score; checked explicitly so that no input, NaN included, loops)
    if (rerun || __ballot(over) == 0) break;
    rerun = true;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      m_ref[rb] = m_ref[rb] == -INFINITY ? m_ref[rb] : fmaxf(m_ref[rb], tm[rb]);
      l_part[rb] = 0.f;
      t_max[rb] = -INFINITY;
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) O[rb][cb][i] = 0.f;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();   // the maxima are read before red is written again
    load_idx(k0);
    issue_tile(k0, buf0);
    load_idx(k0 + BN);
  }

  // ---- epilogue: row sums, partial results ---------------------------------
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  constexpr int SROW = LRB;                         // padded staging row (bytes), bf16
  static_assert((BM / 2) * SROW <= BUF, "O staging must fit in the tile buffers");
  auto srow = [&](int row) -> uint8_t* { return row < BM / 2 ? buf0 + row * SROW : buf1 + (row - BM / 2) * SROW; };
  __syncthreads();   // every wave is done with the tile buffers and red
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const float s = group_sum(l_part[rb]);
    if (lg == 0) red(16 * rb + l16)[w] = s;
  }
  {
    // lane holds row 32 rb + l32, columns col0 + 32 cb + 8 q + 4 half + (0..3)
    const int col0 = w * CPW;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint8_t* dst = srow(32 * rb + l32) + (col0 + 32 * cb + 8 * q + 4 * half) * 2;
          const f32x16& o = O[rb][cb];
          u32x2 v;
          v[0] = pack_bf16(o[4 * q], o[4 * q + 1]);
          v[1] = pack_bf16(o[4 * q + 2], o[4 * q + 3]);
          *reinterpret_cast<u32x2*>(dst) = v;
        }
  }
  __syncthreads();
  const long long gro = (long long)g * p.rows;
  if (w == 0 && lg == 0) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int row = 16 * rb + l16;
      if (row < nrows) {
        const f32x4 s4 = *reinterpret_cast<const f32x4*>(red(row));
        *reinterpret_cast<f32x2*>(p.ws_ml + (gro + idx0 + row) * 2) = f32x2{m_ref[rb], (s4[0] + s4[1]) + (s4[2] + s4[3])};
      }
    }
  }
  {
    constexpr int V16 = DV * 2 / 16;                // 16-byte chunks per row
    constexpr int NST = BM * V16 / 256;
    uint8_t* wso = reinterpret_cast<uint8_t*>(p.ws_o);
    u32x4 v[NST];
#pragma unroll
    for (int j = 0; j < NST; ++j) {
      const int e = tid + 256 * j;
      v[j] = *reinterpret_cast<const u32x4*>(srow(e / V16) + 16 * (e % V16));
    }
#pragma unroll
    for (int j = 0; j < NST; ++j) {
      const int e = tid + 256 * j;
      const int row = e / V16;
      if (row < nrows) st16(wso + ((gro + idx0 + row) * DV) * 2 + 16 * (e % V16), v[j]);
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
namespace {
SplitArgs split_args(const AbsorbedLaunch& q) {
  SplitArgs a{};
  a.q_lat = (const uint16_t*)q.q_lat; a.q_pe = (const uint16_t*)q.q_pe;
  a.c_kv = (const uint16_t*)q.c_kv; a.k_pe = (const uint16_t*)q.k_pe;
  a.off = q.off_dev; a.off0 = q.off0; a.kv1 = q.kv1;
  a.ws_o = (uint16_t*)q.ws_o; a.ws_ml = q.ws_ml;
  a.B = q.B; a.L = q.L; a.H = q.H; a.rows = q.L * q.H;
  a.row_tiles = q.plan.row_tiles; a.chunk = q.plan.chunk; a.n_items = q.plan.n_items;
  a.sl2 = q.scale * 1.4426950408889634f;
  // L2 prefetch window: an XCD's 32 CUs run 32 / row_tiles distinct splits at a
  // time, each with pf_ahead tiles (72 KB) in flight; about row_tiles tiles keeps
  // that near 2 MB of its 4 MB L2
  a.pf_ahead = std::min(16, std::max(2, a.row_tiles));
  return a;
}
unsigned grid_of(int n_items) { return (unsigned)(((n_items + kXcds - 1) / kXcds) * kXcds); }
}  // namespace

hipError_t absorbed_attn_bf16(const AbsorbedLaunch& q, hipStream_t st) {
  const SplitArgs a = split_args(q);
  if (q.r != 512) return hipErrorInvalidValue;
  const dim3 grid(grid_of(a.n_items));
  switch (q.rope) {
    case 0:  hipLaunchKernelGGL((absorbed_split_kernel<0, false>), grid, dim3(256), 0, st, a); break;
    case 64: hipLaunchKernelGGL((absorbed_split_kernel<64, false>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t absorbed_attn_sparse(const AbsorbedLaunch& q, const int32_t* sel, const int32_t* koff_dev, int koff0,
                                int kvt1, hipStream_t st) {
  SplitArgs a = split_args(q);
  a.sel = sel; a.koff = koff_dev; a.koff0 = koff0; a.kvt1 = kvt1;
  if (q.r != 512) return hipErrorInvalidValue;
  const dim3 grid(grid_of(a.n_items));
  switch (q.rope) {
    case 0:  hipLaunchKernelGGL((absorbed_split_kernel<0, true>), grid, dim3(256), 0, st, a); break;
    case 64: hipLaunchKernelGGL((absorbed_split_kernel<64, true>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
