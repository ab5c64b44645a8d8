// attn.hip -- split-KV attention kernels of libmla and their combine passes.
//
// The two MLA routes (pages: "One guard, 110x off the verify step", section
// "The defect"):
//   absorbed     : every (row, head) pair of a sequence is a query of width
//                  r + rope = [q_lat | q_pe] against the shared keys
//                  [c_kv | k_pe]; the values are c_kv itself (multi-query
//                  attention with a single shared key/value head).  Its bf16
//                  and fp8 split kernels are in split_absorbed.hip; this file
//                  holds its float32 kernel and its merge + up-projection;
//   materialised : each head attends over its own expanded K [T, H, n+rope]
//                  and V [T, H, v] (the bf16 kernel below, float32 kernel).
// Positions of a sequence are cut into splits; each workgroup takes query
// rows x one split and leaves unnormalised partial results (o, running max m,
// running sum l, base-2 logits) in a workspace.  A second pass merges the
// splits with a log-sum-exp combine; on the absorbed route it also applies
// the value up-projection W_UV (bf16 MFMA).  No floating-point atomics: the
// result is bitwise reproducible.
//
// bf16 workgroup layout (256 threads = 4 waves, 64 rows, 64-key tiles):
//   scores  S^T[64 keys x 64 rows] as 2x2 blocks of 32x32; wave (wk, wr)
//           computes keys 32wk.., rows 32wr.. with the query block held in
//           registers (B operand) and keys streamed from LDS (A operand);
//   softmax base-2, against a fixed reference per row (the row's maximum
//           over the first tile of the split that gives it finite scores);
//           a split in which a later score exceeds its reference by more
//           than 2^64 runs again with raised references, so O is never
//           rescaled inside the tile loop;
//   PV      O^T[DV x 64 rows]: wave w owns columns w*DV/4..; P (bf16) comes
//           from LDS, V^T fragments are read transposed from the row-major
//           tile with ds_read_b64_tr_b16.
// LDS holds two tile buffers (tile t is computed while tile t+1 is copied in
// by direct-to-LDS loads issued between the score MFMAs), P and small
// exchange arrays.

#include <algorithm>
#include <type_traits>

#include "mla_device.h"
#include "internal.h"

namespace mla {

// ---------------------------------------------------------------------------
// bf16 MFMA split-KV attention
// ---------------------------------------------------------------------------
struct AttnArgs {
  const uint16_t* qa;   // query part a: [B, L, H, DA]
  const uint16_t* qb;   // query part b: [B, L, H, DR]
  const uint16_t* ka;   // keys, row for position p at ka + p*ka_ks + head*ka_hs
  const uint16_t* vv;   // values, row for position p at vv + p*vv_ks + head*vv_hs
  long long ka_ks, ka_hs, vv_ks, vv_hs;
  const int32_t* off;   // [B+1] device offsets
  int off0, kv1;        // B == 1: off[0] and off[1] - off[0]
  float* ws_o;          // [G][rows_total][DV] unnormalised partial sums (float32)
  float* ws_ml;         // [G][rows_total][2]
  int B, L, H;
  int rows_slot;        // query rows per (sequence, head) = L
  int row_tiles;        // ceil(rows_slot / 64)
  int chunk;            // positions per split (multiple of 64)
  int n_items;
  int rows_total;       // L*H
  float sl2;            // scale * log2(e)
};

// Headroom of the fixed softmax reference (log2 units): P = 2^(s - m) <= 2^64.
constexpr float kRefSlack = 64.f;

// DA: width of query part a (q_nope, n); DR: query part b width (rope); DV:
// value width.
//
// Tiles of 64 positions are copied global -> LDS by direct-to-LDS loads (each
// wave instruction fills 1 KB of LDS, lane l at +16*l), double-buffered: tile
// t+1 is in flight while tile t is computed.  LDS rows carry one 16-byte pad
// chunk (row stride = 16 * (chunks + 1) bytes, 144 mod 256 or 16 mod 256), so
// consecutive rows start in different banks and every LDS address is a
// per-lane base plus a compile-time offset.  The PV product reads V^T
// fragments straight from the row-major tile with ds_read_b64_tr_b16 (lane l
// of each 16-lane group receives column l%16 of the 4 rows its group
// addressed), so there is no transposed copy of V.
template <int DA, int DR, int DV>
__global__ __launch_bounds__(256, 1) void attn_bf16_kernel(AttnArgs p) {
  constexpr int D = DA + DR;
  constexpr int BM = 64, BN = 64;
  constexpr int DCH = D / 16;             // 16-wide k steps of the score MFMA
  constexpr int KCH = D / 8;              // 16-byte chunks per key row
  constexpr int VCH = DV / 8;
  constexpr int KRB = (KCH + 1) * 16;     // padded LDS row stride (bytes)
  constexpr int VRB = (VCH + 1) * 16;
  constexpr int KBYTES = BN * KRB;
  constexpr int VBYTES = BN * VRB;
  constexpr int BUF = KBYTES + VBYTES;
  constexpr int KINST = KCH + 1;          // direct-load wave instructions per key tile (64 slots each)
  constexpr int VINST = VCH + 1;
  constexpr int PRB = 9 * 16;             // P row: 64 keys (8 chunks) + pad
  constexpr int CPW = DV / 4;             // value columns per wave
  constexpr int NCB = CPW / 32;           // 32-column MFMA blocks per wave
  static_assert(D % 16 == 0 && DV % 128 == 0, "unsupported geometry");

  // two distinct LDS objects, so that alias analysis can tell the tile being
  // read from the tile being copied in (no spurious waits on the copy)
  __shared__ __attribute__((aligned(1024))) uint8_t buf0[BUF];
  __shared__ __attribute__((aligned(1024))) uint8_t buf1[BUF];
  __shared__ __attribute__((aligned(16))) uint8_t pl[BM * PRB];
  __shared__ __attribute__((aligned(16))) float red[BM * 4];   // per row: 4 partial values (2 key halves x 2 lane halves)

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  // work-item decode, kept in scalar registers (uniform over the workgroup)
  const int item = __builtin_amdgcn_readfirstlane(xcd_item(blockIdx.x, p.n_items));
  if (item >= p.n_items) return;
  const int rt = __builtin_amdgcn_readfirstlane(item % p.row_tiles);
  const int tmp = __builtin_amdgcn_readfirstlane(item / p.row_tiles);
  const int hs = __builtin_amdgcn_readfirstlane(tmp % p.H);   // head
  const int g = __builtin_amdgcn_readfirstlane(tmp / p.H);
  // the split is the same for the whole workgroup: keep its bounds in scalar registers
  // (one sequence: its start and length come from the host, no load of the offsets)
  int b = 0, ps = g, off_b = p.off0, Kv = p.kv1;
  if (p.B > 1) {
    const SplitPos sp = decode_split(g, p.off, p.B, p.chunk);
    b = __builtin_amdgcn_readfirstlane(sp.b);
    ps = __builtin_amdgcn_readfirstlane(sp.s);
    off_b = __builtin_amdgcn_readfirstlane(p.off[b]);
    Kv = __builtin_amdgcn_readfirstlane(p.off[b + 1]) - off_b;
  }
  const long long p0 = off_b;
  const int k0 = __builtin_amdgcn_readfirstlane(ps * p.chunk);
  const int k1 = __builtin_amdgcn_readfirstlane(min(Kv, k0 + p.chunk));
  auto visible = [&](int i) -> int { return Kv - p.L + i + 1; };   // positions query row i may see
  const int idx0 = rt * BM;
  const int nrows = min(BM, p.rows_slot - idx0);

  const uint16_t* kab = p.ka + (long long)hs * p.ka_hs;
  const uint16_t* vvb = p.vv + (long long)hs * p.vv_hs;

  // ---- tile copy: global -> LDS --------------------------------------------
  // Each wave instruction fills 1 KB of LDS: slot (64 j + lane) -> (row, chunk)
  // of the padded tile; the pad slot of a row copies any valid chunk.
  // Load instructions of one wave for a tile, numbered 0..NLW-1, so that the
  // copy can be spread over the score MFMAs instead of stalling the wave.
  constexpr int NLW_K = (KINST + 3) / 4;
  constexpr int NLW_V = (VINST + 3) / 4;
  constexpr int NLW = NLW_K + NLW_V;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  auto issue_part = [&](int t0, uint8_t* kdst, int x) {
    if (x < NLW_K) {
      const int j = wu + 4 * x;
      if (j < KINST) {
        const int pos = 64 * j + lane;            // chunk slot in the tile
        const int key = pos / (KCH + 1);
        int ch = pos - key * (KCH + 1);
        if (ch == KCH) ch = 0;                    // pad slot: any valid chunk
        const long long kk = p0 + min(t0 + key, k1 - 1);
        __builtin_amdgcn_global_load_lds(kab + kk * p.ka_ks + 8 * ch,
                                         (__attribute__((address_space(3))) void*)(kdst + 1024 * j), 16, 0, 0);
      }
    } else {
      const int j = wu + 4 * (x - NLW_K);
      if (j < VINST) {
        uint8_t* vdst = kdst + KBYTES;
        const int pos = 64 * j + lane;
        const int key = pos / (VCH + 1);
        int ch = pos - key * (VCH + 1);
        if (ch == VCH) ch = 0;
        const long long kk = p0 + min(t0 + key, k1 - 1);
        __builtin_amdgcn_global_load_lds(vvb + kk * p.vv_ks + 8 * ch,
                                         (__attribute__((address_space(3))) void*)(vdst + 1024 * j), 16, 0, 0);
      }
    }
  };
  auto issue_tile = [&](int t0, uint8_t* kdst) {
#pragma unroll
    for (int x = 0; x < NLW; ++x) issue_part(t0, kdst, x);
  };

  // ---- score-phase identity: wave (wk, wr), query row rq of the tile -------
  const int wk = w & 1, wr = w >> 1;
  const int rq = 32 * wr + l32;
  const bool rq_ok = rq < nrows;
  int kend = 0;   // positions this row may see within the split (relative to sequence start)
  u32x4 qf[DCH];

  issue_tile(k0, buf0);   // first tile in flight while the queries load
  kend = min(k1, visible(idx0 + rq));
  // positions every row of the tile may see (rows are in increasing query order)
  const int kfull = __builtin_amdgcn_readfirstlane(min(k1, visible(idx0)));
  {
    const int i = idx0 + rq;
    const long long flat = ((long long)b * p.L + i) * p.H + hs;
#pragma unroll
    for (int c = 0; c < DCH; ++c) {
      const int dim = 16 * c + 8 * half;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (rq_ok) {
        if (dim < DA) v = ld16(p.qa + flat * DA + dim);
        else v = ld16(p.qb + flat * DR + (dim - DA));
      }
      qf[c] = v;
    }
  }

  // ---- running state ------------------------------------------------------
  float m_run = -INFINITY, l_run = 0.f;   // score layout: row rq, this wave's key half
  float t_max = -INFINITY;                 // this lane's largest logit of row rq in the split
  float m_all = -INFINITY;                 // reference of row `lane` (the same in every wave)
  f32x16 O[2][NCB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) O[rb][cb][i] = 0.f;

  // per-lane LDS offsets (bytes) within a buffer; the rest are immediates
  const int qk_off = (32 * wk + l32) * KRB + 16 * half;                   // + 32 c
  const int G = lane >> 4, s16 = lane & 15;
  const int tr_off = (8 * (G >> 1) + (s16 >> 2)) * VRB                    // key part
                     + (w * CPW + 16 * (G & 1) + 4 * (s16 & 3)) * 2;      // column part
  const int pa_off = l32 * PRB + 16 * half;                               // + rb*32*PRB + 32 kc

  auto row_max_all = [&](int row) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(&red[row * 4]);
    return fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3]));
  };
  // one 64-position tile: scores from `cur`, copy of the next tile into `nxt`
  auto step = [&](int t0, const uint8_t* cur, uint8_t* nxt, bool pf) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // (A) tile t visible; PV(t-1) done, so the other buffer and pl are free
    // The next tile is copied unconditionally (branch-free code keeps the LDS
    // wait counts exact): past the end of the split every row clamps to the
    // last position and lands in the idle buffer, which nothing reads again.
    const uint8_t* kt = cur;
    const uint8_t* vt = kt + KBYTES;

    // ---- scores: S^T block [32 keys x 32 rows] --------------------------
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    {
      // key fragments are read 4 steps ahead of their MFMA; the sched-group
      // barriers pin an LDS-read / MFMA interleave so reads stay in flight
      constexpr int PF = 8;
      const uint8_t* kq = kt + qk_off;
      u32x4 ka[PF];
#pragma unroll
      for (int c = 0; c < PF; ++c) ka[c] = *reinterpret_cast<const u32x4*>(kq + 32 * c);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < DCH; ++c) {
        const u32x4 a = ka[c % PF];
        if (c + PF < DCH) ka[c % PF] = *reinterpret_cast<const u32x4*>(kq + 32 * (c + PF));
        acc = mfma32(a, qf[c], acc);
        // next tile's copy, spread over the score MFMAs (NLW instructions)
        if (pf) {
#pragma unroll
          for (int x = (c * NLW) / DCH; x < ((c + 1) * NLW) / DCH; ++x) issue_part(t0 + BN, nxt, x);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the read of step c+PF ahead of MFMA c
      }
    }
    // acc[i] = q.k for key t0 + 32 wk + 8 (i >> 2) + 4 half + (i & 3), row rq.
    // Tiles inside every row's causal range (all but the last ones of a split)
    // skip the key mask (a uniform branch).
    float s[16];
    if (t0 + BN <= kfull) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = acc[i];
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = t0 + 32 * wk + 8 * (i >> 2) + 4 * half + (i & 3);
        s[i] = key < kend ? acc[i] : -INFINITY;
      }
    }
    float pmax = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
    pmax = fmaxf(pmax, fmaxf(fmaxf(fmaxf(s[8], s[9]), fmaxf(s[10], s[11])), fmaxf(fmaxf(s[12], s[13]), fmaxf(s[14], s[15]))));
    pmax *= p.sl2;   // base-2 logits: scale * log2(e) * q.k
    // Fixed reference per row: P = 2^(s - m) with m the row's maximum over the
    // first tile that gives it finite scores.  P (bf16) and O, l (fp32) keep
    // their relative precision at any magnitude, so later scores may exceed m
    // by up to kRefSlack (P <= 2^64) and O is never rescaled inside the loop;
    // a split in which some row exceeds that runs again with raised references
    // (checked after its last tile).  P is computed here against the current
    // reference; the first tile, which sets the references, recomputes it
    // below.  A row without a finite reference uses 0: its masked keys give
    // 2^-inf = 0.
    uint8_t* prow = pl + rq * PRB + 64 * wk + 8 * half;
    auto write_p = [&](float mref, float* psum) {
      const float mb = mref == -INFINITY ? 0.f : mref;
      float e[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) e[i] = __builtin_amdgcn_exp2f(fmaf(s[i], p.sl2, -mb));
      // the row sum adds the bf16 weights that PV uses, so that numerator and
      // denominator carry the same rounding (exact for a row led by one key)
      float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x2 v;
        v[0] = pack_bf16(e[4 * q + 0], e[4 * q + 1]);
        v[1] = pack_bf16(e[4 * q + 2], e[4 * q + 3]);
        *reinterpret_cast<u32x2*>(prow + 16 * q) = v;
        ps0 = add_bf16x2(v[0], ps0);
        ps1 = add_bf16x2(v[1], ps1);
      }
      *psum = ps0 + ps1;
    };
    float psum;
    write_p(m_run, &psum);
    t_max = fmaxf(t_max, pmax);
    // A row sees a prefix of the split's positions, so every row with finite
    // scores in the split has them in its first tile: the references are set
    // there from the tile's row maxima.  Later tiles publish only P; whether
    // some row outgrew its reference is decided once, after the last tile.
    auto row_max = [&](int row) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(&red[row * 4]);
      return fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3]));
    };
    if (t0 == k0) {
      red[rq * 4 + wk * 2 + half] = pmax;   // maximum over this lane's 16 keys
      lds_barrier();  // (B) P and partial maxima visible (the next tile's copy stays in flight)
      // Every wave decides for all 64 rows (lane = row) from the same partial
      // maxima with the same arithmetic, so the decision is uniform over the
      // workgroup and the branch (with its barrier) is taken by all waves or by none.
      const float tm_all = row_max(lane);
      if (__ballot(m_all == -INFINITY && tm_all != -INFINITY) != 0) {
        // first finite scores of some rows (O is still 0 there): their reference
        // is this tile's maximum; the other rows recompute the same P
        m_all = (m_all == -INFINITY) ? tm_all : m_all;
        if (m_run == -INFINITY) m_run = row_max(rq);
        write_p(m_run, &psum);
        lds_barrier();  // (C) recomputed P visible
      }
    } else {
      lds_barrier();  // (B) P visible
    }
    l_run += psum;

    // ---- PV: O[64 rows x CPW] for this wave's columns ----------------------
    {
      const uint8_t* pa = pl + pa_off;
      const uint8_t* vb = vt + tr_off;
      // V^T fragment for step (kc, cb): two transposing reads of 4 keys each
      auto vfrag = [&](int kc, int cb) {
        u32x4 bv;
#pragma unroll
        for (int ld = 0; ld < 2; ++ld) {
          const uint8_t* src = vb + (16 * kc + 4 * ld) * VRB + 64 * cb;
          const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(src));
          const u32x2 rr = __builtin_bit_cast(u32x2, r);
          bv[2 * ld] = rr[0];
          bv[2 * ld + 1] = rr[1];
        }
        return bv;
      };
      constexpr int NSTEP = (BN / 16) * NCB;
      constexpr int VPF = 3;   // V^T fragments in flight (steps ahead)
      u32x4 a[BN / 16][2];     // P fragments of every k step (read ahead with the first V step of that k)
      u32x4 vq[VPF];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) a[0][rb] = *reinterpret_cast<const u32x4*>(pa + rb * 32 * PRB);
#pragma unroll
      for (int st = 0; st < VPF; ++st) {
        if (st < NSTEP) {
          if (st > 0 && st % NCB == 0) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
              a[st / NCB][rb] = *reinterpret_cast<const u32x4*>(pa + rb * 32 * PRB + 32 * (st / NCB));
          }
          vq[st] = vfrag(st / NCB, st % NCB);
        }
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
        __builtin_amdgcn_sched_barrier(0);   // later steps' reads stay ahead of this step's MFMAs
      }
    }
  };
  // Tiles go in pairs (one per buffer); an odd tile count skips the second
  // step of the last pair.  No copy follows the last tile.
  for (;;) {
    for (int t0 = k0; t0 < k1; t0 += 2 * BN) {
      step(t0, buf0, buf1, t0 + BN < k1);
      if (t0 + BN < k1) step(t0 + BN, buf1, buf0, t0 + 2 * BN < k1);
    }
    // Did some row's scores exceed its reference by more than 2^kRefSlack (P up
    // to 2^kRefSlack keeps fp32 and bf16 exact in relative terms)?  Then its
    // P, O and l may have overflowed: raise every reference to the row's
    // maximum over the whole split and run the split again.  The second pass
    // cannot trigger another, since its references bound every score.
    __syncthreads();   // every wave is done with red and the tile buffers
    red[rq * 4 + wk * 2 + half] = t_max;
    lds_barrier();
    const float tm_all = row_max_all(lane);
    if (__ballot(m_all != -INFINITY && tm_all > m_all + kRefSlack) == 0) break;
    m_all = fmaxf(m_all, tm_all);
    m_run = fmaxf(m_run, row_max_all(rq));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();   // the maxima are read before red is written again
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) O[rb][cb][i] = 0.f;
    l_run = 0.f;
    t_max = -INFINITY;
    issue_tile(k0, buf0);
  }

  // ---- epilogue: row sums, partial results ---------------------------------
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  constexpr int PB = 4;                             // bytes per partial element (float32)
  constexpr int SROW = DV * PB + 16;                // padded staging row (bytes)
  static_assert((BM / 2) * SROW <= BUF, "O staging must fit in the tile buffers");
  // rows 0..31 staged in buf0, rows 32..63 in buf1
  auto srow = [&](int row) -> uint8_t* { return row < BM / 2 ? buf0 + row * SROW : buf1 + (row - BM / 2) * SROW; };
  __syncthreads();   // every wave is done with the tile buffers and red
  red[rq * 4 + wk * 2 + half] = l_run;   // sum over this lane's keys
  {
    // lane holds row 32 rb + l32, columns col0 + 32 cb + 8 q + 4 half + (0..3)
    const int col0 = w * CPW;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint8_t* dst = srow(32 * rb + l32) + (col0 + 32 * cb + 8 * q + 4 * half) * PB;
          const f32x16& o = O[rb][cb];
          *reinterpret_cast<f32x4*>(dst) = f32x4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
        }
  }
  __syncthreads();
  const long long gro = (long long)g * p.rows_total;
  if (wk == 0 && half == 0 && rq_ok) {
    const int prow = hs * p.rows_slot + idx0 + rq;
    p.ws_ml[(gro + prow) * 2 + 0] = m_run;
    const f32x4 a = *reinterpret_cast<const f32x4*>(&red[rq * 4]);
    p.ws_ml[(gro + prow) * 2 + 1] = (a[0] + a[1]) + (a[2] + a[3]);
  }
  {
    // rows out with 16-byte coalesced stores, all LDS reads first
    constexpr int V16 = DV * PB / 16;               // 16-byte chunks per row
    constexpr int NST = BM * V16 / 256;
    static_assert(BM * V16 % 256 == 0, "whole rounds of stores");
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
      if (row < nrows) {
        const int prow = hs * p.rows_slot + idx0 + row;
        st16(wso + ((gro + prow) * DV) * PB + 16 * (e % V16), v[j]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// float32 split-KV attention (VALU).  One workgroup per (split, head slot,
// query row); same partial-result format as the bf16 kernel.
// ---------------------------------------------------------------------------
struct AttnArgsF32 {
  const float* qa; const float* qb;
  const float* ka; const float* kb; const float* vv;
  long long ka_ks, ka_hs, kb_ks, kb_hs, vv_ks, vv_hs;
  int DA, DR, DV;
  const int32_t* off;
  float* ws_o; float* ws_ml;
  int B, L, H, hpr, rows_slot, head_slots, chunk, n_items, rows_total;
  float sl2;
};

constexpr int kF32MaxD = 1152;   // q width limit of the float32 kernel (DA + DR)
constexpr int kF32MaxDV = 1024;

__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgsF32 p) {
  constexpr int NT = 256, BN = 256;
  __shared__ float q[kF32MaxD];
  __shared__ float sc[BN];
  __shared__ float redm[NT / 64];
  const int tid = threadIdx.x;
  const int item = blockIdx.x;
  if (item >= p.n_items) return;
  const int idx = item % p.rows_slot;
  const int tmp = item / p.rows_slot;
  const int hs = tmp % p.head_slots;
  const int g = tmp / p.head_slots;
  const SplitPos sp = decode_split(g, p.off, p.B, p.chunk);
  const int b = sp.b;
  const long long p0 = p.off[b];
  const int Kv = p.off[b + 1] - p.off[b];
  const int k0 = sp.s * p.chunk;
  const int k1 = min(Kv, k0 + p.chunk);
  const int i = idx / p.hpr;
  const int h = hs + idx % p.hpr;
  const long long flat = ((long long)b * p.L + i) * p.H + h;
  const int kend = min(k1, Kv - p.L + i + 1);
  for (int d = tid; d < p.DA + p.DR; d += NT)
    q[d] = d < p.DA ? p.qa[flat * p.DA + d] : p.qb[flat * p.DR + d - p.DA];
  float o[kF32MaxDV / NT];
  for (int x = 0; x < kF32MaxDV / NT; ++x) o[x] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  __syncthreads();
  for (int t0 = k0; t0 < kend; t0 += BN) {
    const int key = t0 + tid;
    float s = -INFINITY;
    if (key < kend) {
      const float* kr = p.ka + (p0 + key) * p.ka_ks + hs * p.ka_hs;
      const float* kr2 = p.kb + (p0 + key) * p.kb_ks + hs * p.kb_hs;
      float a = 0.f;
      for (int d = 0; d < p.DA; ++d) a = fmaf(q[d], kr[d], a);
      for (int d = 0; d < p.DR; ++d) a = fmaf(q[p.DA + d], kr2[d], a);
      s = a * p.sl2;
    }
    float mx = s;
    for (int d = 32; d >= 1; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d, 64));
    if ((tid & 63) == 0) redm[tid >> 6] = mx;
    __syncthreads();
    float tmax = redm[0];
    for (int x = 1; x < NT / 64; ++x) tmax = fmaxf(tmax, redm[x]);
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    sc[tid] = key < kend ? __builtin_amdgcn_exp2f(s - m_new) : 0.f;
    __syncthreads();
    const int nk = min(BN, kend - t0);
    float ps = 0.f;
    for (int t = 0; t < nk; ++t) ps += sc[t];
    l_run = l_run * alpha + ps;
    m_run = m_new;
    for (int x = 0; x * NT + tid < p.DV; ++x) {
      const int c = x * NT + tid;
      float a = o[x] * alpha;
      for (int t = 0; t < nk; ++t) a = fmaf(sc[t], p.vv[(p0 + t0 + t) * p.vv_ks + hs * p.vv_hs + c], a);
      o[x] = a;
    }
    __syncthreads();
  }
  const long long prow = (long long)g * p.rows_total + hs * p.rows_slot + idx;
  if (tid == 0) {
    p.ws_ml[prow * 2 + 0] = m_run;
    p.ws_ml[prow * 2 + 1] = l_run;
  }
  for (int x = 0; x * NT + tid < p.DV; ++x) p.ws_o[prow * p.DV + x * NT + tid] = o[x];
}

// ---------------------------------------------------------------------------
// Combine passes.
// ---------------------------------------------------------------------------
// Merge weights of the splits of one partial row: w_s = 2^(m_s - M) / sum_s 2^(m_s - M) l_s.
__device__ __forceinline__ void merge_stats(const float* __restrict__ ml, long long stride_rows, int S,
                                            float* M_out, float* inv_out) {
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, ml[s * stride_rows * 2]);
  float den = 0.f;
  for (int s = 0; s < S; ++s) {
    const float m = ml[s * stride_rows * 2];
    if (m != -INFINITY) den += __builtin_amdgcn_exp2f(m - M) * ml[s * stride_rows * 2 + 1];
  }
  *M_out = M;
  *inv_out = 1.f / den;
}

__device__ __forceinline__ float ld_part(const float* p, long long i) { return p[i]; }
__device__ __forceinline__ float ld_part(const uint16_t* p, long long i) { return bf16_to_f32(p[i]); }

// out[b,i,h,:] = sum_s w_s o_s  (materialised route; float32 or bf16 partials).
template <typename PT>
__global__ __launch_bounds__(256) void combine_kernel(const PT* __restrict__ ws_o, const float* __restrict__ ws_ml,
                                                      const int32_t* __restrict__ off, int B, int L, int H, int DV,
                                                      int chunk, float* __restrict__ out) {
  const int row = blockIdx.x;          // (b, i, h) flat
  const int h = row % H, i = (row / H) % L, b = row / (H * L);
  const int rows_total = L * H;
  const int prow = h * L + i;
  int g0, S;
  seq_splits(b, off, chunk, &g0, &S);
  const float* ml = ws_ml + ((long long)g0 * rows_total + prow) * 2;
  float M, inv;
  merge_stats(ml, rows_total, S, &M, &inv);
  for (int c = threadIdx.x; c < DV; c += blockDim.x) {
    float a = 0.f;
    for (int s = 0; s < S; ++s) {
      const float m = ml[(long long)s * rows_total * 2];
      if (m == -INFINITY) continue;
      a = fmaf(__builtin_amdgcn_exp2f(m - M), ld_part(ws_o, ((long long)(g0 + s) * rows_total + prow) * DV + c), a);
    }
    out[(long long)row * DV + c] = a * inv;
  }
}

// Absorbed route, float32: o_lat = merged latent, out = o_lat . W_UV[h].
__global__ __launch_bounds__(256) void combine_upproj_f32_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
                                                                 const int32_t* __restrict__ off, int B, int L, int H,
                                                                 int R, int V, int chunk, const float* __restrict__ w_uv,
                                                                 float* __restrict__ out) {
  __shared__ float ol[1024];
  const int row = blockIdx.x;
  const int h = row % H, i = (row / H) % L, b = row / (H * L);
  const int rows_total = L * H;
  const int prow = i * H + h;
  int g0, S;
  seq_splits(b, off, chunk, &g0, &S);
  const float* ml = ws_ml + ((long long)g0 * rows_total + prow) * 2;
  float M, inv;
  merge_stats(ml, rows_total, S, &M, &inv);
  for (int c = threadIdx.x; c < R; c += blockDim.x) {
    float a = 0.f;
    for (int s = 0; s < S; ++s) {
      const float m = ml[(long long)s * rows_total * 2];
      if (m == -INFINITY) continue;
      a = fmaf(__builtin_amdgcn_exp2f(m - M), ws_o[((long long)(g0 + s) * rows_total + prow) * R + c], a);
    }
    ol[c] = a * inv;
  }
  __syncthreads();
  const float* wh = w_uv + (long long)h * R * V;
  for (int e = threadIdx.x; e < V; e += blockDim.x) {
    float a = 0.f;
    for (int c = 0; c < R; ++c) a = fmaf(ol[c], wh[(long long)c * V + e], a);
    out[(long long)row * V + e] = a;
  }
}

// Absorbed route, bf16: merge of the splits and up-projection in one pass,
//   out[b,i,h,:] = (sum_s w_s o_s[b,i,h,:]) . W_UV[h],  w_s = 2^(m_s - M) / den,
// from the bf16 partial sums.  Work item = (sequence b, head h, 16 query rows,
// 64 output columns), the column tile varying fastest so that the items that
// read the same partial sums run on one XCD and share its L2.  The W_UV tile
// [r x 64] goes global -> LDS with direct loads while the partial sums come
// into registers, 16 16-byte loads per lane in flight.  Wave w merges rows
// w, w+NW, .. (RPW of them; lane l: latent columns 8l..8l+7) in float32,
// stores the merged latent as a bf16 pair hi + lo (hi = bf16(x),
// lo = bf16(x - hi)) and multiplies both with 16x16x32 MFMAs, W fragments
// read transposed from LDS.
struct MergeUpArgs {
  const uint16_t* ws_o; const float* ws_ml; const int32_t* off;
  const uint16_t* w_uv;   // [H][R][V]
  float* out;             // [B][L][H][V]
  int B, L, H, V, chunk;
  int S1;                 // splits of the sequence when B == 1
  int MTS, CT, n_items;   // row tiles of 16 per sequence, column tiles of 64, items
};

// NW waves (4 or 8), RPW query rows per wave (NW RPW <= 16 rows per tile).
// With eight waves twice the loads are in flight per CU; the product then
// splits K over wave halves (waves 4..7 hand their partial sums over in LDS).
// WSTREAM: the W_UV tile is loaded with the streaming hint, for launches in which
// one workgroup reads each W_UV line (one sequence, one row tile); with more, the
// workgroups of the other sequences and row tiles re-read it from L2.
template <int R, int RPW, int NW, bool WSTREAM>
__global__ __launch_bounds__(64 * NW, 1) void merge_upproj_kernel(MergeUpArgs p) {
  static_assert(R / 8 == kWave, "one lane per 8 latent columns");
  constexpr int WRB = 64 * 2 + 16;            // W row: 64 bf16 + pad (bytes)
  constexpr int WCH = WRB / 16;               // 16-byte slots per W row (8 data + 1 pad)
  constexpr int WINST = R * WCH / kWave;      // direct-load wave instructions for the tile
  constexpr int ARB = R * 2 + 16;             // A row: R bf16 + pad
  constexpr int SB = (NW == 8 ? 16 : 32) / RPW;   // splits per row per round of loads
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  static_assert(NW * RPW <= 16, "a row tile of at most 16 rows");
  static_assert(WINST % NW == 0 && kWave % SB == 0, "tile split over the waves; rounds inside a 64-split window");
  __shared__ __attribute__((aligned(1024))) uint8_t wt[R * WRB];
  __shared__ __attribute__((aligned(16))) uint8_t at[2][16 * ARB];
  __shared__ __attribute__((aligned(16))) f32x4 kpart[NW == 8 ? 4 * kWave : 1];   // K-half sums of waves 4..7

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int item = xcd_item(blockIdx.x, p.n_items);
  if (item >= p.n_items) return;
  const int ct = item % p.CT;
  int tmp = item / p.CT;
  const int mt = tmp % p.MTS;
  tmp /= p.MTS;
  const int h = tmp % p.H, b = tmp / p.H;
  const int rows_total = p.L * p.H;
  const int i0 = 16 * mt;
  const int mrows = min(16, p.L - i0);

  // ---- W_UV tile -> LDS (slot j*64 + lane = (row, 16-byte chunk); pad slots load chunk 0)
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const uint16_t* wsrc = p.w_uv + (long long)h * R * p.V + ct * 64;
  auto issue_w = [&]() {
#pragma unroll
    for (int x = 0; x < WINST / NW; ++x) {
      const int j = wu + NW * x;
      const int pos = kWave * j + lane;
      const int row = pos / WCH;
      int ch = pos - row * WCH;
      if (ch == WCH - 1) ch = 0;
      __builtin_amdgcn_global_load_lds(wsrc + (long long)row * p.V + 8 * ch,
                                       (__attribute__((address_space(3))) void*)(wt + 1024 * j), 16, 0,
                                       WSTREAM ? 2 : 0);
    }
  };

  // splits of sequence b: g0 .. g0+S-1 (one sequence: given by the host)
  int g0 = 0, S = p.S1;
  if (p.B > 1) {
    seq_splits(b, p.off, p.chunk, &g0, &S);
    g0 = __builtin_amdgcn_readfirstlane(g0);
    S = __builtin_amdgcn_readfirstlane(S);
  }
  // rows of this wave: w + NW rr for rr < nr (row m of the tile is query row i0 + m)
  const int nr = min(RPW, mrows > wu ? (mrows - wu + NW - 1) / NW : 0);
  const uint16_t* obase = p.ws_o + (long long)g0 * rows_total * R + 8 * lane;
  // flat partial-sum row of each slot; slots past this wave's rows repeat its last row
  // (a wave without rows reads nothing)
  int prow[RPW];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) prow[rr] = (i0 + (nr > 0 ? wu + NW * min(rr, nr - 1) : 0)) * p.H + h;

  float o[RPW][8];
  float M[RPW], inv[RPW], wl[RPW];   // wl: merge weight of split 64*(s0/64) + lane
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
#pragma unroll
    for (int c = 0; c < 8; ++c) o[rr][c] = 0.f;
    M[rr] = -INFINITY; inv[rr] = 0.f; wl[rr] = 0.f;
  }

  // (max, sum) of split `lane` for every row: loaded before the partial sums, so that
  // waiting for them does not wait for the partial sums
  float mv[RPW], lv[RPW];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    mv[rr] = -INFINITY;
    lv[rr] = 0.f;
    if (nr > 0 && lane < S) {
      const f32x2 ml = *reinterpret_cast<const f32x2*>(p.ws_ml + ((long long)(g0 + lane) * rows_total + prow[rr]) * 2);
      mv[rr] = ml[0];
      lv[rr] = ml[1];
    }
  }

  for (int s0 = 0; s0 < (nr > 0 ? S : 0); s0 += SB) {
    // one round of loads: splits s0 .. s0+SB-1 of every row of the wave (clamped; the
    // surplus gets weight 0)
    u32x4 v[RPW][SB];
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr)
#pragma unroll
      for (int j = 0; j < SB; ++j)
        v[rr][j] = ld16(obase + ((long long)min(s0 + j, S - 1) * rows_total + prow[rr]) * R);
    if (s0 == 0) issue_w();
    if (s0 % kWave == 0) {
      // merge statistics of every row (first round) and the weights of the splits
      // s0 + lane (the window of this round)
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr) {
        if (s0 == 0) {
          float mx = mv[rr], den = mv[rr] == -INFINITY ? 0.f : lv[rr];
          for (int t0 = kWave; t0 < S; t0 += kWave) {   // more than 64 splits
            const int s = t0 + lane;
            float m = -INFINITY, l = 0.f;
            if (s < S) {
              const f32x2 ml = *reinterpret_cast<const f32x2*>(p.ws_ml + ((long long)(g0 + s) * rows_total + prow[rr]) * 2);
              m = ml[0];
              l = ml[1];
            }
            const float nm = fmaxf(mx, m);   // running (max, sum) over this lane's splits
            if (nm != -INFINITY)
              den = (mx == -INFINITY ? 0.f : den * __builtin_amdgcn_exp2f(mx - nm)) +
                    (m == -INFINITY ? 0.f : l * __builtin_amdgcn_exp2f(m - nm));
            mx = nm;
          }
          float wmx = mx;
#pragma unroll
          for (int d = 32; d >= 1; d >>= 1) wmx = fmaxf(wmx, __shfl_xor(wmx, d, kWave));
          den = (mx == -INFINITY) ? 0.f : den * __builtin_amdgcn_exp2f(mx - wmx);
#pragma unroll
          for (int d = 32; d >= 1; d >>= 1) den += __shfl_xor(den, d, kWave);
          M[rr] = wmx;
          inv[rr] = 1.f / den;
        }
        const int s = s0 + lane;
        float m = mv[rr];
        if (s0 > 0) m = s < S ? p.ws_ml[((long long)(g0 + s) * rows_total + prow[rr]) * 2] : -INFINITY;
        wl[rr] = (m == -INFINITY || rr >= nr) ? 0.f : __builtin_amdgcn_exp2f(m - M[rr]) * inv[rr];
      }
    }
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr)
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        // weight of split s0 + j, read from its lane of the window (uniform lane index)
        const float wf = (s0 + j < S) ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl[rr]), (s0 + j) % kWave)) : 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          o[rr][2 * c] = fmaf(wf, bf16_lo(v[rr][j][c]), o[rr][2 * c]);
          o[rr][2 * c + 1] = fmaf(wf, bf16_hi(v[rr][j][c]), o[rr][2 * c + 1]);
        }
      }
  }

  if (nr == 0) issue_w();

  // ---- merged latent -> LDS as hi + lo bf16 (rows without a query row are zero)
#pragma unroll
  for (int rr = 0; rr < 16 / NW; ++rr) {
    const int m = wu + NW * rr;
    u32x4 hi = {0u, 0u, 0u, 0u}, lo = {0u, 0u, 0u, 0u};
    if (rr < RPW && rr < nr) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float x0 = o[rr < RPW ? rr : 0][2 * c], x1 = o[rr < RPW ? rr : 0][2 * c + 1];
        hi[c] = pack_bf16(x0, x1);
        lo[c] = pack_bf16(x0 - bf16_lo(hi[c]), x1 - bf16_hi(hi[c]));
      }
    }
    st16(at[0] + m * ARB + 16 * lane, hi);
    st16(at[1] + m * ARB + 16 * lane, lo);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's part of the W tile has landed
  __syncthreads();

  // ---- out tile [16 rows x 64 columns]: wave w -> columns 16 cb .. + 15 (cb = w % 4),
  // k steps kh R / 64 .. of the half kh = w / 4 (eight waves; all of them with four)
  const int r16 = lane & 15, G = lane >> 4;
  const int cb = wu & 3, kh = NW == 8 ? wu >> 2 : 0;
  constexpr int NKS = (R / 32) / (NW / 4);
  const uint8_t* wb = wt + (8 * G + (r16 >> 2)) * WRB + (16 * cb + 4 * (r16 & 3)) * 2;
  const uint8_t* ab0 = at[0] + r16 * ARB + 16 * G;
  const uint8_t* ab1 = at[1] + r16 * ARB + 16 * G;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < NKS; ++kk) {
    const int ks = kh * NKS + kk;
    u32x4 bv;
#pragma unroll
    for (int ld = 0; ld < 2; ++ld) {
      const v4i16 rr = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16*)(wb + (32 * ks + 4 * ld) * WRB));
      const u32x2 r2 = __builtin_bit_cast(u32x2, rr);
      bv[2 * ld] = r2[0];
      bv[2 * ld + 1] = r2[1];
    }
    acc = mfma16(*reinterpret_cast<const u32x4*>(ab0 + 64 * ks), bv, acc);
    acc = mfma16(*reinterpret_cast<const u32x4*>(ab1 + 64 * ks), bv, acc);
  }
  if (NW == 8) {
    if (kh == 1) kpart[cb * kWave + lane] = acc;
    __syncthreads();
    if (kh == 1) return;
    const f32x4 o = kpart[cb * kWave + lane];
#pragma unroll
    for (int x = 0; x < 4; ++x) acc[x] += o[x];
  }
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int m = 4 * G + x;
    if (m < mrows)
      __builtin_nontemporal_store(acc[x], &p.out[(((long long)b * p.L + i0 + m) * p.H + h) * p.V + ct * 64 + 16 * cb + r16]);
  }
}

// Absorbed route, bf16, few (sequence, row, head) triples: merge and
// up-projection with one work item per (sequence b, query row i, head h, 64
// output columns).  The four waves share the splits of the row (wave w takes
// splits w, w + 4, ...; lane l latent columns 8l .. 8l + 7), the four partial
// latents meet in LDS in a fixed order, and the merged latent (float32) is
// multiplied by the W_UV tile [r x 64] on the VALU (thread t: the 8 columns
// 8 (t % 8) .., latent indices 16 (t / 8) .. + 15, all 16 weight loads of 16
// bytes issued before the first product; the 32 slices summed in LDS).  Items of
// the same (b, h, column tile) are adjacent, so they share their W_UV tile in
// one XCD's L2.  Used when the head-tile merge would leave most CUs idle.
template <int R>
__global__ __launch_bounds__(256) void merge_rows_kernel(MergeUpArgs p) {
  static_assert(R / 8 == kWave, "one lane per 8 latent columns");
  __shared__ __attribute__((aligned(16))) float part[4][R];
  __shared__ __attribute__((aligned(16))) float ocol[32][64 + 4];
  static_assert(R == 32 * 16, "32 slices of 16 latent indices");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int item = xcd_item(blockIdx.x, p.n_items);
  if (item >= p.n_items) return;
  // item = ((b * H + h) * CT + ct) * L + i
  const int i = item % p.L;
  int tmp = item / p.L;
  const int ct = tmp % p.CT;
  tmp /= p.CT;
  const int h = tmp % p.H, b = tmp / p.H;
  const int rows_total = p.L * p.H;
  const int prow = i * p.H + h;
  int g0 = 0, S = p.S1;
  if (p.B > 1) {
    seq_splits(b, p.off, p.chunk, &g0, &S);
    g0 = __builtin_amdgcn_readfirstlane(g0);
    S = __builtin_amdgcn_readfirstlane(S);
  }
  const float* ml = p.ws_ml + ((long long)g0 * rows_total + prow) * 2;
  const uint16_t* obase = p.ws_o + ((long long)g0 * rows_total + prow) * R + 8 * lane;
  // The partial sums of this wave's first NPRE splits (w, w + 4, ..) and this
  // thread's W_UV slice are requested before the merge statistics, which they
  // do not depend on: one memory round trip instead of two.
  constexpr int NPRE = 16;
  u32x4 vpre[NPRE];
#pragma unroll
  for (int j = 0; j < NPRE; ++j)
    if (w + 4 * j < S) vpre[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(obase + (long long)(w + 4 * j) * rows_total * R));
  const int cg = tid & 7, ks = tid >> 3;
  const uint16_t* wsrc = p.w_uv + (long long)h * R * p.V + (long long)(16 * ks) * p.V + ct * 64 + 8 * cg;
  u32x4 wv[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) wv[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wsrc + (long long)k * p.V));
  // merge statistics, M = max_s m_s, den = sum_s 2^(m_s - M) l_s, lane-strided
  // over the splits; every wave computes them (the same order, the same values)
  float M, inv;
  {
    float mx = -INFINITY;
    for (int s = lane; s < S; s += kWave) mx = fmaxf(mx, ml[(long long)s * rows_total * 2]);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d, kWave));
    float den = 0.f;
    for (int s = lane; s < S; s += kWave) {
      const float m = ml[(long long)s * rows_total * 2];
      if (m != -INFINITY) den += __builtin_amdgcn_exp2f(m - mx) * ml[(long long)s * rows_total * 2 + 1];
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) den += __shfl_xor(den, d, kWave);
    M = mx;
    inv = 1.f / den;
  }
  // this wave's splits: 8 latent columns per lane, float32, in split order
  float o[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) o[c] = 0.f;
#pragma unroll
  for (int j = 0; j < NPRE; ++j) {
    const int s = w + 4 * j;
    if (s < S) {
      const float m = ml[(long long)s * rows_total * 2];
      const float wt = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M) * inv;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        o[2 * c] = fmaf(wt, bf16_lo(vpre[j][c]), o[2 * c]);
        o[2 * c + 1] = fmaf(wt, bf16_hi(vpre[j][c]), o[2 * c + 1]);
      }
    }
  }
  int s = w + 4 * NPRE;
  for (; s + 12 < S; s += 16) {   // four splits of this wave in flight
    u32x4 v[4];
    float wt[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(obase + (long long)(s + 4 * j) * rows_total * R));
      const float m = ml[(long long)(s + 4 * j) * rows_total * 2];
      wt[j] = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M) * inv;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        o[2 * c] = fmaf(wt[j], bf16_lo(v[j][c]), o[2 * c]);
        o[2 * c + 1] = fmaf(wt[j], bf16_hi(v[j][c]), o[2 * c + 1]);
      }
  }
  for (; s < S; s += 4) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(obase + (long long)s * rows_total * R));
    const float m = ml[(long long)s * rows_total * 2];
    const float wt = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M) * inv;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      o[2 * c] = fmaf(wt, bf16_lo(v[c]), o[2 * c]);
      o[2 * c + 1] = fmaf(wt, bf16_hi(v[c]), o[2 * c + 1]);
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) part[w][8 * lane + c] = o[c];
  __syncthreads();
  // merged latent row (waves' sums in a fixed order) times W_UV[h][:, 64 ct ..]
  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int kk = 16 * ks + k;
    const float x = (part[0][kk] + part[1][kk]) + (part[2][kk] + part[3][kk]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      acc[2 * c] = fmaf(x, bf16_lo(wv[k][c]), acc[2 * c]);
      acc[2 * c + 1] = fmaf(x, bf16_hi(wv[k][c]), acc[2 * c + 1]);
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) ocol[ks][8 * cg + c] = acc[c];
  __syncthreads();
  if (tid < 64) {
    float t = 0.f;
    for (int k = 0; k < 32; ++k) t += ocol[k][tid];
    p.out[(((long long)b * p.L + i) * p.H + h) * p.V + ct * 64 + tid] = t;
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static inline unsigned grid_xcd(int n_items) { return (unsigned)(((n_items + kXcds - 1) / kXcds) * kXcds); }

template <int DA, int DR, int DV>
static hipError_t launch_attn(const AttnArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((attn_bf16_kernel<DA, DR, DV>), dim3(grid_xcd(a.n_items)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t materialized_attn_bf16(const MaterializedLaunch& q, hipStream_t st) {
  AttnArgs a{};
  const int D = q.n + q.rope;
  a.qa = (const uint16_t*)q.q_nope; a.qb = (const uint16_t*)q.q_pe;
  a.ka = (const uint16_t*)q.k; a.ka_ks = (long long)q.H * D; a.ka_hs = D;
  a.vv = (const uint16_t*)q.v; a.vv_ks = (long long)q.H * q.v_dim; a.vv_hs = q.v_dim;
  a.off = q.off_dev; a.off0 = q.off0; a.kv1 = q.kv1; a.ws_o = (float*)q.ws_o; a.ws_ml = q.ws_ml;
  a.B = q.B; a.L = q.L; a.H = q.H; a.rows_slot = q.L;
  a.row_tiles = q.plan.row_tiles; a.chunk = q.plan.chunk; a.n_items = q.plan.n_items;
  a.rows_total = q.L * q.H; a.sl2 = q.scale * 1.4426950408889634f;
  // The kernel sees the query as [q_nope | q_pe] of width n + rope and K rows
  // of the same width; DA = n, DR = rope.
#define MLA_MAT(N, RP, VD) \
  if (q.n == N && q.rope == RP && q.v_dim == VD) return launch_attn<N, RP, VD>(a, st);
  MLA_MAT(128, 64, 128) MLA_MAT(128, 64, 256) MLA_MAT(192, 64, 128) MLA_MAT(192, 64, 256)
  MLA_MAT(256, 64, 128) MLA_MAT(256, 64, 256) MLA_MAT(128, 0, 128) MLA_MAT(256, 0, 256)
  MLA_MAT(192, 0, 256) MLA_MAT(128, 0, 256) MLA_MAT(256, 0, 128) MLA_MAT(192, 0, 128)
#undef MLA_MAT
  return hipErrorInvalidValue;
}

bool materialized_bf16_supported(int n, int rope, int v) {
  const bool nn = (n == 128 || n == 192 || n == 256);
  const bool rr = (rope == 0 || rope == 64);
  const bool vv = (v == 128 || v == 256);
  return nn && rr && vv;
}

hipError_t attn_f32(const AbsorbedLaunch* qa, const MaterializedLaunch* qm, hipStream_t st) {
  AttnArgsF32 a{};
  if (qa) {
    const AbsorbedLaunch& q = *qa;
    a.qa = (const float*)q.q_lat; a.qb = (const float*)q.q_pe;
    a.ka = (const float*)q.c_kv; a.ka_ks = q.r; a.ka_hs = 0;
    a.kb = (const float*)q.k_pe; a.kb_ks = q.rope; a.kb_hs = 0;
    a.vv = (const float*)q.c_kv; a.vv_ks = q.r; a.vv_hs = 0;
    a.DA = q.r; a.DR = q.rope; a.DV = q.r;
    a.off = q.off_dev; a.ws_o = (float*)q.ws_o; a.ws_ml = q.ws_ml;
    a.B = q.B; a.L = q.L; a.H = q.H; a.hpr = q.H; a.rows_slot = q.L * q.H; a.head_slots = 1;
    a.chunk = q.plan.chunk; a.rows_total = q.L * q.H; a.sl2 = q.scale * 1.4426950408889634f;
    a.n_items = q.plan.n_splits * a.head_slots * a.rows_slot;
  } else {
    const MaterializedLaunch& q = *qm;
    const int D = q.n + q.rope;
    a.qa = (const float*)q.q_nope; a.qb = (const float*)q.q_pe;
    a.ka = (const float*)q.k; a.ka_ks = (long long)q.H * D; a.ka_hs = D;
    a.kb = (const float*)q.k + q.n; a.kb_ks = (long long)q.H * D; a.kb_hs = D;
    a.vv = (const float*)q.v; a.vv_ks = (long long)q.H * q.v_dim; a.vv_hs = q.v_dim;
    a.DA = q.n; a.DR = q.rope; a.DV = q.v_dim;
    a.off = q.off_dev; a.ws_o = (float*)q.ws_o; a.ws_ml = q.ws_ml;
    a.B = q.B; a.L = q.L; a.H = q.H; a.hpr = 1; a.rows_slot = q.L; a.head_slots = q.H;
    a.chunk = q.plan.chunk; a.rows_total = q.L * q.H; a.sl2 = q.scale * 1.4426950408889634f;
    a.n_items = q.plan.n_splits * a.head_slots * a.rows_slot;
  }
  if (a.DA + a.DR > kF32MaxD || a.DV > kF32MaxDV) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_f32_kernel, dim3(a.n_items), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t combine_materialized(const MaterializedLaunch& q, mla_dtype_t dt, float* out, hipStream_t st) {
  (void)dt;   // the materialised route keeps float32 partials for both input types
  hipLaunchKernelGGL(combine_kernel<float>, dim3(q.B * q.L * q.H), dim3(256), 0, st, (const float*)q.ws_o,
                     (const float*)q.ws_ml, q.off_dev, q.B, q.L, q.H, q.v_dim, q.plan.chunk, out);
  return hipGetLastError();
}

hipError_t combine_upproj(const AbsorbedLaunch& q, mla_dtype_t dt, float* out, hipStream_t st) {
  if (dt == kF32) {
    hipLaunchKernelGGL(combine_upproj_f32_kernel, dim3(q.B * q.L * q.H), dim3(256), 0, st,
                       (const float*)q.ws_o, (const float*)q.ws_ml, q.off_dev, q.B, q.L, q.H, q.r, q.v_dim,
                       q.plan.chunk, (const float*)q.w_uv, out);
    return hipGetLastError();
  }
  if (q.r != 512 || q.v_dim % 64 != 0) return hipErrorInvalidValue;
  MergeUpArgs a{};
  a.ws_o = (const uint16_t*)q.ws_o; a.ws_ml = q.ws_ml; a.off = q.off_dev;
  a.w_uv = (const uint16_t*)q.w_uv; a.out = out;
  a.B = q.B; a.L = q.L; a.H = q.H; a.V = q.v_dim; a.chunk = q.plan.chunk;
  a.S1 = q.plan.n_splits;
  a.MTS = (q.L + 15) / 16; a.CT = q.v_dim / 64;
  const long long items = (long long)q.B * q.H * a.MTS * a.CT;
  if (items > INT32_MAX) return hipErrorInvalidValue;
  a.n_items = (int)items;
  // few (sequence, head) pairs: one item per query row instead, the splits shared by the waves
  const long long row_items = (long long)q.B * q.H * q.L * a.CT;
  if (items < kNumCUs && row_items <= INT32_MAX) {
    a.n_items = (int)row_items;
    hipLaunchKernelGGL((merge_rows_kernel<512>), dim3(grid_xcd(a.n_items)), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  // eight waves, one or two query rows each
  const dim3 grid(grid_xcd(a.n_items));
  const bool once = q.B == 1 && a.MTS == 1;   // each W_UV line read by one workgroup
  if (q.L <= 8 && once) hipLaunchKernelGGL((merge_upproj_kernel<512, 1, 8, true>), grid, dim3(512), 0, st, a);
  else if (q.L <= 8) hipLaunchKernelGGL((merge_upproj_kernel<512, 1, 8, false>), grid, dim3(512), 0, st, a);
  else if (once) hipLaunchKernelGGL((merge_upproj_kernel<512, 2, 8, true>), grid, dim3(512), 0, st, a);
  else hipLaunchKernelGGL((merge_upproj_kernel<512, 2, 8, false>), grid, dim3(512), 0, st, a);
  return hipGetLastError();
}

}  // namespace mla
