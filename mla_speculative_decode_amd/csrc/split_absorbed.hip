// split_absorbed.hip -- the split-KV kernels of the absorbed MLA route over the
// latent cache (pages: "One guard, 110x off the verify step", section "The
// defect": attend directly against the compressed latent and accumulate in
// latent space).
//
// The absorbed route is multi-query attention with one shared key/value head:
// every (row, head) pair of a sequence is a query of width 512 + rope against
// the keys [c_kv | k_pe], and the values are c_kv itself.  A workgroup takes 64
// query rows x one split of the sequence's positions and leaves unnormalised
// partial results (latent sums in bf16, the row's base-2 reference and sum in
// float32) for the merge pass.
//
// bf16 cache (absorbed_split_kernel): eight waves, two per SIMD, in two roles
// that form a pipeline over tiles of 32 positions.  The scoring waves hold the
// query block in registers and compute S^T with 16x16x32 bf16 MFMAs, then the
// weights P = 2^(s - m) against a fixed reference per row (the row's maximum
// over the split's first tile; a split whose later scores exceed it by more
// than 2^64 runs again with raised references, so O is never rescaled); the PV
// waves accumulate O^T = V^T P^T with 32x32x16 MFMAs, V^T read transposed from
// the row-major tile (ds_read_b64_tr_b16), and copy the next tile in.  Scores
// of tile k, PV of tile k - 1 and the copy of tile k + 1 share a phase.
//
// fp8 cache (absorbed_split_f8_kernel): the scores on the scaled fp8 matrix
// cores with the queries block-quantised in the kernel; 32 query rows per
// workgroup, two workgroups per CU.
//
// Both have a selected-position form (SEL) that runs over a per-sequence list
// of cache positions instead of all of them.

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
  const uint8_t* c8;       // fp8 form: E4M3 codes [T, 512 + DR] (latent | rope)
  const float* s8;         // fp8 form: one power-of-two scale per position [T]
  const uint8_t* q8;       // fp8 form: the E4M3 query blocks (kQ8TileBytes per 32 rows), or null: quantise here
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
  int pf_lines;            // fp8 form: 128-byte lines of a tile each row tile prefetches
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

// ---------------------------------------------------------------------------
// The split over the fp8 form of the latent cache (E4M3 codes of each
// position's row [c_kv | k_pe] with one power-of-two scale per position).
//
//   scores  on the scaled fp8 MFMA (16x16x128): the query block is quantised
//           once, in the prologue, to E4M3 with one power-of-two scale per
//           (row, 32-wide block of the key dimension), the smallest with every
//           |q| <= 448 x scale; the keys' codes come straight from LDS, with
//           their position's scale as the A-side block scale.  The rope part
//           is one more k step whose upper half is zero.
//   softmax base 2 against a fixed reference per row (the row's maximum over
//           the split's first tile; a split whose later scores exceed it by
//           more than 2^64 runs again with raised references); each weight is
//           then multiplied by its key's scale (a power of two, so bf16(P) x 2^k
//           is exact) before it goes to LDS, and the row sums add the unscaled
//           weights.
//   PV      O^T += V^T P^T on bf16 32x32x16 MFMAs; a V^T fragment is one
//           transposed byte read (ds_read_b64_tr_b8: 8 keys of one column)
//           widened to bf16 (codes are exact in bf16), the scale having gone
//           into P.
// A workgroup takes 32 query rows (two workgroups share a CU, so one's softmax
// and barriers overlap the other's MFMAs).  LDS: two tile buffers, each 64
// latent code rows (512 bytes, unpadded, 16-byte chunks XOR-swizzled by row),
// 64 rope code rows and the tile's 64 scales; then P; the epilogue stages O
// in a tile buffer.
// ---------------------------------------------------------------------------
namespace {
// Direct global -> LDS copy (BYTES = 16 or 4 per lane) written as inline asm:
// the compiler then does not track it, so it adds no waits of its own before
// LDS reads of other buffers.  The kernel waits for its copies itself (vmcnt)
// before the barrier that publishes a tile.  M0 is written here and used by
// nothing else in the kernel.
template <int BYTES>
__device__ __forceinline__ void dma(const void* gsrc, const void* lds_dst) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds_dst);
  if (BYTES == 16)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "s"(m) : "memory");
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(gsrc), "s"(m) : "memory");
}
// the same with a uniform 64-bit base (scalar registers) and a per-lane 32-bit
// byte offset: the address needs no 64-bit vector arithmetic
template <int BYTES>
__device__ __forceinline__ void dma_sv(const void* sbase, uint32_t voff, const void* lds_dst) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds_dst);
  if (BYTES == 16)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m) : "memory");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(m) : "memory");
}
// the same with the LDS destination given as an LDS address (uniform)
template <int BYTES>
__device__ __forceinline__ void dma_sv_to(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds_addr);
  if (BYTES == 16)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m) : "memory");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(m) : "memory");
}
template <int BYTES>
__device__ __forceinline__ void dma_to(const void* gsrc, uint32_t lds_addr) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds_addr);
  if (BYTES == 16)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "s"(m) : "memory");
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(gsrc), "s"(m) : "memory");
}
// the same with an immediate byte offset on the global address; the
// instruction adds it to the LDS address as well, so M0 is set OFF lower
template <int OFF>
__device__ __forceinline__ void dma16_off(const void* gsrc, uint32_t lds_addr) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds_addr - OFF);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%2" ::"v"(gsrc), "s"(m), "i"(OFF)
               : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}
// mfma16_f8 with B's scale in byte `sel` of scale_b (sel known once the caller's
// loop is unrolled)
__device__ __forceinline__ f32x4 mfma16_f8_sel(i32x8 a, i32x8 b, f32x4 c, int scale_a, int scale_b, int sel) {
  switch (sel) {
    case 0: return mfma16_f8<0>(a, b, c, scale_a, scale_b);
    case 1: return mfma16_f8<1>(a, b, c, scale_a, scale_b);
    case 2: return mfma16_f8<2>(a, b, c, scale_a, scale_b);
    default: return mfma16_f8<3>(a, b, c, scale_a, scale_b);
  }
}
// two E4M3 codes (bytes 2 HI, 2 HI + 1 of w) -> packed bf16 (exact)
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
}  // namespace

// Q8: the queries come quantised (the fold's E4M3 query block, p.q8).
template <int DR, bool SEL, bool Q8>
__global__ __launch_bounds__(256, 2) void absorbed_split_f8_kernel(SplitArgs p) {
  constexpr int DA = 512, DV = 512;
  constexpr int BM = 32, BN = 64;
  constexpr int NRB = BM / 16;            // 16-row blocks of the score layout
  constexpr int DW = DA + DR;             // codes per cached position
  constexpr int ROPE = BN * DA;           // rope region: 64 rows of DR bytes after the latent rows
  constexpr int SOFF = ROPE + BN * DR;    // the tile's 64 scales follow
  constexpr int BUF = SOFF + BN * 4;
  constexpr int NLI = BN / 2;             // latent copy instructions per tile (two rows each)
  constexpr int NRI = BN * DR / 1024;     // rope copy instructions per tile (16 rows each)
  constexpr int KS = DA / 128;            // 128-wide score k steps over the latent part
  constexpr int NQ = KS + (DR > 0 ? 1 : 0);
  constexpr int PRB = 9 * 16;             // P row: 64 keys (8 chunks) + one chunk holding 4 exchange floats
  constexpr int CPW = DV / 4;             // value columns per wave
  constexpr int NCB = CPW / 32;           // 32-column MFMA blocks per wave
  constexpr int NLW = NLI / 4;            // latent copies per wave per tile
  constexpr int NC = NLW / 2;             // ... of which these go with the scores, the rest with PV
  constexpr int SROW = DV * 2 + 8;        // epilogue staging row (bf16; 8 mod 256 bytes)
  constexpr int QGS = 17 * 16, QHS = 81 * 16, QFS = 164 * 16;   // query staging strides (16-byte slots 1, 1, 4 mod 16)
  constexpr int QSS = 68;                 // scale slots per (rb, ks): 64 lanes + 4 (banks 4 ks + 16 j + l % 16)
  constexpr int QBYTES = NRB * KS * QFS + (DR > 0 ? NRB * kWave * 16 : 0);   // query codes
  static_assert(DR == 0 || DR == 64, "rope width 0 or 64");
  static_assert(BUF % 16 == 0, "layout");
  static_assert(QHS >= 4 * QGS && QFS >= 2 * QHS, "staging strides");
  static_assert(QBYTES <= BUF && NRB * NQ * QSS * 4 <= BM * PRB, "query codes fit in a tile buffer, their scales in pl");
  static_assert(BM * SROW <= BUF, "O staging fits in a tile buffer");
  static_assert(2 * BUF + BM * PRB + 4 * kWave <= 160 * 1024 / 2, "two workgroups per CU");
  static_assert(NRI <= 4 && NLW % 2 == 0, "copy layout");

  // separate arrays, so that the compiler can tell the tile being read from the
  // one the direct loads are filling
  __shared__ __attribute__((aligned(1024))) uint8_t buf0[BUF];
  __shared__ __attribute__((aligned(1024))) uint8_t buf1[BUF];
  __shared__ __attribute__((aligned(16))) uint8_t pl[BM * PRB];
  __shared__ uint32_t pfd[kWave];   // landing slot of the L2 prefetch (never read)
  auto red = [&](int row) -> float* { return reinterpret_cast<float*>(pl + row * PRB + 128); };

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int half = lane >> 5, l32 = lane & 31;
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
  long long p0 = off_b;
  int Kt = Kv;
  if (SEL) {
    p0 = p.B > 1 ? (long long)__builtin_amdgcn_readfirstlane(p.koff[b]) : (long long)p.koff0;
    Kt = p.B > 1 ? __builtin_amdgcn_readfirstlane(p.koff[b + 1]) - (int)p0 : p.kvt1;
  }
  const int sel0 = off_b;
  const int k0 = __builtin_amdgcn_readfirstlane(ps * p.chunk);
  const int k1 = __builtin_amdgcn_readfirstlane(min(Kv, k0 + p.chunk));
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
    int lo = 0, hi = Kv;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (p.sel[sel0 + mid] < bound) lo = mid + 1; else hi = mid;
    }
    return lo;
  };
  int sidx = 0;
  auto load_idx = [&](int t0) {
    if (SEL) sidx = min(max(p.sel[sel0 + min(t0 + lane, k1 - 1)], 0), Kt - 1);
  };
  const int idx0 = rt * BM;
  const int nrows = min(BM, p.rows - idx0);
  const uint8_t* cbase = p.c8 + p0 * DW;
  const float* sbase = p.s8 + p0;

  // ---- tile copy: global -> LDS ----------------------------------------------
  // Latent rows of 512 codes, unpadded, 16-byte chunk c of row r stored at
  // chunk c ^ 2 (r & 7).  A ds_read_b128 serves the 16 lanes of a half-wave
  // whose lane bits 2 ^ 3 ^ 4 agree, a transposed read a half-wave: with this
  // swizzle the 16 lanes of a score-fragment read, and the 8 rows x 2 chunks of
  // a transposed V read, each touch every bank once.  One wave
  // instruction fills two rows (lane l: row 2 j + l / 32, stored chunk l % 32),
  // every lane active; the rope parts (64 bytes a row, chunk c at c ^ (r & 3))
  // take one instruction per 16 rows, the scales one per tile.
  // This wave's latent pairs are j = wu + 4 x: lane l copies row r = 2 j + l / 32
  // = 8 x + (2 wu + l / 32), whose swizzle 2 (r & 7) is 2 (2 wu + l / 32) for every x.
  const int lrow = 2 * wu + (lane >> 5);                   // row of the pair (x = 0) for this lane
  const int lsw0 = 16 * ((lane & 31) ^ (2 * lrow)), lsw1 = lsw0;
  const int rrow = lane >> 2, rpc = lane & 3;              // rope copy: row in the 16, stored chunk
  auto pos_of = [&](int t0, int key) -> int {              // cache position of tile row `key` (per lane)
    return SEL ? __shfl(sidx, key, kWave) : min(t0 + key, k1 - 1);
  };
  // Dense tiles address the codes from the tile's first position (a scalar
  // base) plus a per-lane 32-bit offset (rows clamped to the split's last);
  // selected positions are arbitrary and keep the 64-bit per-lane form.
  auto issue_latent = [&](int t0, uint8_t* kdst, int x) {
    if (SEL) {
      const int pos = pos_of(t0, 8 * x + lrow);
      dma<16>(cbase + (long long)pos * DW + ((x & 1) ? lsw1 : lsw0), kdst + 1024 * (wu + 4 * x));
    } else {
      const int row = min(8 * x + lrow, k1 - 1 - t0);
      dma_sv<16>(cbase + (long long)t0 * DW, (uint32_t)(row * DW + ((x & 1) ? lsw1 : lsw0)), kdst + 1024 * (wu + 4 * x));
    }
  };
  auto issue_rope = [&](int t0, uint8_t* kdst, int j) {
    const int r = 16 * j + rrow;
    if (SEL) {
      const int pos = pos_of(t0, r);
      dma<16>(cbase + (long long)pos * DW + DA + 16 * (rpc ^ (r & 3)), kdst + ROPE + 1024 * j);
    } else {
      const int row = min(r, k1 - 1 - t0);
      dma_sv<16>(cbase + (long long)t0 * DW, (uint32_t)(row * DW + DA + 16 * (rpc ^ (r & 3))), kdst + ROPE + 1024 * j);
    }
  };
  // the tile's 64 scales (lane j: key j)
  auto issue_scales = [&](int t0, uint8_t* kdst) {
    if (SEL) dma<4>(sbase + pos_of(t0, lane), kdst + SOFF);
    else dma_sv<4>(sbase + t0, (uint32_t)(4 * min(lane, k1 - 1 - t0)), kdst + SOFF);
  };
  // copy x of this wave (x < NLW: latent pair wu + 4 x; NLW: its rope block or
  // the scales)
  auto issue_part = [&](int t0, uint8_t* kdst, int x) {
    if (x < NLW) issue_latent(t0, kdst, x);
    else if (wu < NRI) issue_rope(t0, kdst, wu);
    else if (wu == 3) issue_scales(t0, kdst);
  };
  auto issue_tile = [&](int t0, uint8_t* kdst) {
#pragma unroll
    for (int x = 0; x <= NLW; ++x) issue_part(t0, kdst, x);
    if (NRI == 4 && wu == 0) issue_scales(t0, kdst);
  };
  // barrier over LDS traffic that does not wait for the direct loads in flight
  // (a tile is waited for, with vmcnt, before the barrier that publishes it)
  auto lgkm_barrier = [&]() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  int kend[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int idx = idx0 + min(16 * rb + l16, nrows - 1);
    kend[rb] = min(k1, visible(idx / p.H));
  }
  const int kfull = __builtin_amdgcn_readfirstlane(min(k1, visible(idx0 / p.H)));

  // ---- query block -> E4M3 codes and block scales -----------------------------
  // One thread per (row, 32-wide block of the key dimension): the block's
  // scale 2^e is the smallest with every |q| <= 448 x 2^e, and its codes go to
  // buf1 (idle until the next tile's copy) for the B operand of the score MFMA:
  // lane l = row 16 rb + l % 16 over k = 128 ks + 16 (l / 16) .. (half 0) and
  // 128 ks + 64 + 16 (l / 16) .. (half 1) of fragment (rb, ks < KS).  Block j
  // of step ks thus fills half j / 2 of lane groups 2 (j % 2) and 2 (j % 2) + 1,
  // and group j supplies its scale (an int per lane and step, in pl).  The
  // staging holds 16 bytes per (fragment f, half h, lane group G, lane): at
  // f QFS + h QHS + G QGS + 16 (l % 16), the strides padded so that the 16
  // blocks of a row (ks < 4, j) fall in 16 distinct 16-byte bank slots (slot
  // 4 ks + h + G mod 16) and the 16 lanes of a group read one contiguous 256
  // bytes.  The rope step keeps only its lower halves (at ROPE_OFF + 16 (64 rb
  // + l)); its upper halves and blocks 2, 3 are zero.  Rows past the last query
  // row repeat it (their results are never stored).  A thread's query loads are
  // issued before the first tile's copy, so waiting for them does not wait for
  // the tile.
  i32x8 qf[NRB][NQ];
  int qs[NRB][(NQ + 3) / 4];   // E8M0 scales, step ks in byte ks % 4 of qs[rb][ks / 4]
  if (Q8) {
    // the block quantised by the fold: one copy into buf1, then registers (rows
    // past the last query row: zero codes, scale 2^0)
    static_assert(kQ8TileBytes % 1024 == 0 && kQ8TileBytes <= BUF && NRB == 2 && KS == 4, "query block layout");
    const uint8_t* qt = p.q8 + ((long long)b * p.row_tiles + rt) * kQ8TileBytes;
#pragma unroll
    for (int x = wu; x < kQ8TileBytes / 1024; x += 4) dma<16>(qt + 1024 * x + 16 * lane, buf1 + 1024 * x);
    load_idx(k0);
    issue_tile(k0, buf0);
    load_idx(k0 + BN);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const bool ok = 16 * rb + l16 < nrows;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint8_t* const src = buf1 + 16 * (2 * (KS * rb + ks) * kWave + lane);
        const u32x4 x0 = ok ? ld16(src) : u32x4{0u, 0u, 0u, 0u}, x1 = ok ? ld16(src + 16 * kWave) : u32x4{0u, 0u, 0u, 0u};
        qf[rb][ks] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
      }
      if (DR > 0) {
        const u32x4 x0 = ok ? ld16(buf1 + kQ8RopeOff + 16 * (kWave * rb + lane)) : u32x4{0u, 0u, 0u, 0u};
        qf[rb][NQ - 1] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], 0, 0, 0, 0};
      }
#pragma unroll
      for (int k4 = 0; k4 < (NQ + 3) / 4; ++k4)
        qs[rb][k4] = ok ? *reinterpret_cast<const int*>(buf1 + kQ8ScaleOff + 4 * (kWave * (2 * rb + k4) + lane)) : 0x7f7f7f7f;
    }
    // buf1 is written again only after barrier (A) of the first tile
  } else {
    constexpr int NB = DA / 32 + DR / 32;     // blocks per row
    constexpr int NU = (BM * NB + 255) / 256; // blocks per thread (the last round partial)
    constexpr int ROPE_OFF = NRB * KS * QFS;
    const long long qflat0 = (long long)b * p.rows + idx0;
    u32x4 qv[NU][4];
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = min(tid + 256 * i, BM * NB - 1);
      const int row = u / NB, blk = u - row * NB;
      const long long qrow = qflat0 + min(row, nrows - 1);
      const uint16_t* src = blk >= DA / 32 ? p.q_pe + qrow * DR + 32 * (blk - DA / 32) : p.q_lat + qrow * DA + 32 * blk;
#pragma unroll
      for (int c = 0; c < 4; ++c) qv[i][c] = ld16(src + 8 * c);
    }
    load_idx(k0);
    issue_tile(k0, buf0);   // first tile in flight while the queries are quantised
    load_idx(k0 + BN);
    int* const qsl = reinterpret_cast<int*>(pl);
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = tid + 256 * i;
      if (u < BM * NB) {
        const int row = u / NB, blk = u - row * NB;
        const int e = e4m3_scale_exponent_bf16(absmax32(qv[i]));
        const float sc = __uint_as_float((uint32_t)(e + 127) << 23);
        const int rb = row >> 4, r16 = row & 15;
        const u32x2 c0 = e4m3x8(qv[i][0], sc), c1 = e4m3x8(qv[i][1], sc), c2 = e4m3x8(qv[i][2], sc),
                    c3 = e4m3x8(qv[i][3], sc);
        const u32x4 lo = u32x4{c0[0], c0[1], c1[0], c1[1]}, hi = u32x4{c2[0], c2[1], c3[0], c3[1]};
        if (blk < DA / 32) {
          const int ks = blk >> 2, j = blk & 3;
          uint8_t* const dst = buf1 + (rb * KS + ks) * QFS + (j >> 1) * QHS + 2 * (j & 1) * QGS + 16 * r16;
          st16(dst, lo);
          st16(dst + QGS, hi);
          qsl[QSS * (rb * NQ + ks) + 16 * j + r16] = e + 127;
        } else {
          const int j = blk - DA / 32;
          st16(buf1 + ROPE_OFF + 16 * (64 * rb + 16 * (2 * j) + r16), lo);
          st16(buf1 + ROPE_OFF + 16 * (64 * rb + 16 * (2 * j + 1) + r16), hi);
          qsl[QSS * (rb * NQ + NQ - 1) + 16 * j + r16] = e + 127;
          qsl[QSS * (rb * NQ + NQ - 1) + 16 * (j + 2) + r16] = 127;
        }
      }
    }
    lgkm_barrier();
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint8_t* const src = buf1 + (rb * KS + ks) * QFS + (lane >> 4) * QGS + 16 * l16;
        const u32x4 x0 = ld16(src), x1 = ld16(src + QHS);
        qf[rb][ks] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
      }
      if (DR > 0) {
        const u32x4 x0 = ld16(buf1 + ROPE_OFF + 16 * (64 * rb + lane));
        qf[rb][NQ - 1] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], 0, 0, 0, 0};
      }
#pragma unroll
      for (int k4 = 0; k4 < (NQ + 3) / 4; ++k4) {
        int v = 0;
#pragma unroll
        for (int ks = 4 * k4; ks < min(NQ, 4 * k4 + 4); ++ks) v |= qsl[QSS * (rb * NQ + ks) + lane] << (8 * (ks % 4));
        qs[rb][k4] = v;
      }
    }
    // buf1 and pl are written again only after barrier (A) of the first tile
  }

  // ---- running state (score layout: row 16 rb + l16) -----------------------
  float m_ref[NRB], l_part[NRB], t_max[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) { m_ref[rb] = -INFINITY; l_part[rb] = 0.f; t_max[rb] = -INFINITY; }
  bool rerun = false;
  f32x16 O[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[cb][i] = 0.f;

  // score A fragment of key 16 w + l16: logical chunk 8 ks + lg (+ 4) is stored
  // at (8 ks + lg) ^ 2 (l16 & 7) = (lg ^ 2 (l16 & 7)) ^ 8 ks (chunk bits do not carry)
  const int ka_row = (16 * w + l16) * DA + 16 * (lg ^ (2 * (l16 & 7)));
  const int kr_off = ROPE + (16 * w + l16) * DR + 16 * (lg ^ (l16 & 3));
  const int G = lane >> 4, s16 = lane & 15;
  // V^T fragment of the 32x32x16 MFMA (col 32 cb + l32, keys 16 kc + 8 half ..):
  // source lane s16 of group G reads key 8 (G >> 1) + s16 / 2, 8 codes at column
  // 16 (G & 1) + 8 (s16 & 1); the read hands lane s16 column s16 of the 8 keys.
  // The key's low 3 bits (the swizzle) do not depend on kc.
  // (logical chunk 8 w + 2 cb + (G & 1) is stored at ((8 w + (G & 1)) ^ 2 (key & 7)) ^ 2 cb)
  const int tr_key = 8 * (G >> 1) + (s16 >> 1);
  const int tr_base = tr_key * DA + 8 * (s16 & 1);
  const int tr_sw = (8 * w + (G & 1)) ^ (2 * (tr_key & 7));
  const int pa_off = l32 * PRB + 16 * half;                              // P^T fragment: + 32 kc
  const int pw_off = l16 * PRB + (16 * w + 4 * lg) * 2;                  // + 16 rb PRB

  // Cache lines of tile ta (its codes, then its scales) -> L2 ahead of its
  // copy: the split's row tiles (one XCD, one L2) take pf_lines lines each, tile
  // rt the slice from rt pf_lines, one 4-byte load per line into a dummy LDS slot.
  const int kPfAhead = p.pf_ahead;
  auto prefetch_tile = [&](int ta) {
    if (SEL || ta >= k1 || tid >= p.pf_lines) return;
    const int npos = min(BN, k1 - ta);
    const int code_lines = (npos * DW + 127) / 128;
    const int ln = rt * p.pf_lines + tid;
    const void* src = ln < code_lines ? (const void*)(cbase + (long long)ta * DW + 128 * ln)
                                      : (const void*)(sbase + ta + min(32 * (ln - code_lines), npos - 1));
    if (ln < code_lines + 2) dma<4>(src, pfd);
  };

  auto step = [&](int t0, const uint8_t* cur, uint8_t* nxt, bool pf) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // (A) tile t visible; PV(t-1) done, so the other buffer and pl are free
    if (!SEL && !rerun && wu * kWave < p.pf_lines) {   // the waves holding prefetch lanes
      if (t0 == k0) {
        const int dn = min(kPfAhead, (k1 - 1 - t0) / BN);   // the split's later tiles, up to kPfAhead
        for (int d = 1; d <= dn; ++d) prefetch_tile(t0 + d * BN);
      } else {
        prefetch_tile(t0 + kPfAhead * BN);
      }
    }

    // ---- scores: S^T [16 keys x 32 rows] on the scaled fp8 MFMA ---------------
    f32x4 acc[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
      const int ksc = (int)(__float_as_uint(*reinterpret_cast<const float*>(cur + SOFF + 4 * (16 * w + l16))) >> 23);
      auto afrag = [&](int ks) {
        if (ks == KS) {   // rope: lower half only
          const u32x4 x0 = ld16(cur + kr_off);
          return i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], 0, 0, 0, 0};
        }
        const u32x4 x0 = ld16(cur + (ka_row ^ (16 * 8 * ks)));
        const u32x4 x1 = ld16(cur + (ka_row ^ (16 * (8 * ks + 4))));
        return i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
      };
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < NQ; ++ks) {
        const i32x8 af = afrag(ks);
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
          acc[rb] = mfma16_f8_sel(af, qf[rb][ks], acc[rb], ksc, qs[rb][ks / 4], ks % 4);
        if (pf) {
#pragma unroll
          for (int x = (ks * NC) / NQ; x < ((ks + 1) * NC) / NQ; ++x) issue_latent(t0 + BN, nxt, x);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // acc[rb][i] = q . k for key t0 + 16 w + 4 lg + i, row 16 rb + l16.
    if (t0 + BN > kfull) {   // a tile past some row's causal end (uniform branch)
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (t0 + 16 * w + 4 * lg + i >= kend[rb]) acc[rb][i] = -INFINITY;
    }
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
      t_max[rb] = fmaxf(fmaxf(t_max[rb], fmaxf(acc[rb][0], acc[rb][1])), fmaxf(acc[rb][2], acc[rb][3]));
    // The first tile of the split sets each row's reference (a row sees a prefix
    // of the split's positions, so its first finite scores are in this tile).
    if (t0 == k0 && !rerun) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const float mx = group_max(fmaxf(fmaxf(acc[rb][0], acc[rb][1]), fmaxf(acc[rb][2], acc[rb][3])));
        if (lg == 0) red(16 * rb + l16)[w] = mx * p.sl2;
      }
      lgkm_barrier();
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const f32x4 r4 = *reinterpret_cast<const f32x4*>(red(16 * rb + l16));
        m_ref[rb] = fmaxf(fmaxf(r4[0], r4[1]), fmaxf(r4[2], r4[3]));
      }
    }
    // P = 2^(s - m) in bf16; PV takes P x (key scale), the row sums P
    {
      const f32x4 ksc4 = *reinterpret_cast<const f32x4*>(cur + SOFF + 4 * (16 * w + 4 * lg));
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const float mb = m_ref[rb] == -INFINITY ? 0.f : m_ref[rb];
        float e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = __builtin_amdgcn_exp2f(fmaf(acc[rb][i], p.sl2, -mb));
        const uint32_t v0 = pack_bf16(e[0], e[1]), v1 = pack_bf16(e[2], e[3]);
        l_part[rb] = add_bf16x2(v1, add_bf16x2(v0, l_part[rb]));
        u32x2 v;
        v[0] = pack_bf16(e[0] * ksc4[0], e[1] * ksc4[1]);
        v[1] = pack_bf16(e[2] * ksc4[2], e[3] * ksc4[3]);
        *reinterpret_cast<u32x2*>(pl + pw_off + 16 * rb * PRB) = v;
      }
    }
    lgkm_barrier();  // (B) P visible (the next tile's copy stays in flight)

    // ---- PV: O^T [CPW columns x 32 rows] for this wave's columns --------------
    {
      const uint8_t* pa = pl + pa_off;
      auto vfrag = [&](int kc, int cb) {
        typedef int i32x2 __attribute__((ext_vector_type(2)));
        const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) i32x2*)(cur + tr_base + 16 * kc * DA + 16 * (tr_sw ^ (2 * cb))));
        u32x4 bv;
        bv[0] = e4m3x2_bf16<false>((uint32_t)r[0]);
        bv[1] = e4m3x2_bf16<true>((uint32_t)r[0]);
        bv[2] = e4m3x2_bf16<false>((uint32_t)r[1]);
        bv[3] = e4m3x2_bf16<true>((uint32_t)r[1]);
        return bv;
      };
      constexpr int NSTEP = (BN / 16) * NCB;
      constexpr int VPF = 2;
      u32x4 a[BN / 16];
      u32x4 vq[VPF];
#pragma unroll
      for (int kc = 0; kc < BN / 16; ++kc) a[kc] = *reinterpret_cast<const u32x4*>(pa + 32 * kc);
#pragma unroll
      for (int st = 0; st < VPF; ++st) vq[st] = vfrag(st / NCB, st % NCB);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int st = 0; st < NSTEP; ++st) {
        const int kc = st / NCB, cb = st % NCB;
        const u32x4 bcur = vq[st % VPF];
        const int sn = st + VPF;
        if (sn < NSTEP) vq[st % VPF] = vfrag(sn / NCB, sn % NCB);
        O[cb] = mfma32(bcur, a[kc], O[cb]);   // O^T += V^T P^T
        // the rest of the next tile's copies: latent pairs NC .. NLW - 1, then the
        // rope block / scales, one every other MFMA step
        if (pf && (st & 1) && NC + st / 2 <= NLW) issue_part(t0 + BN, nxt, NC + st / 2);
        if (pf && NRI == 4 && st == 0 && wu == 0) issue_scales(t0 + BN, nxt);
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
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();   // every wave is done with red and the tile buffers
    float tm[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const float mx = group_max(t_max[rb]);
      if (lg == 0) red(16 * rb + l16)[w] = mx * p.sl2;
    }
    lgkm_barrier();
    bool over = false;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const f32x4 r4 = *reinterpret_cast<const f32x4*>(red(16 * rb + l16));
      tm[rb] = fmaxf(fmaxf(r4[0], r4[1]), fmaxf(r4[2], r4[3]));
      over = over || (m_ref[rb] != -INFINITY && tm[rb] > m_ref[rb] + kRefSlack);
    }
    // every wave holds all of the block's rows, so the decision is uniform over
    // the workgroup; checked explicitly so that no input, NaN included, loops
    if (rerun || __ballot(over) == 0) break;
    rerun = true;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      m_ref[rb] = m_ref[rb] == -INFINITY ? m_ref[rb] : fmaxf(m_ref[rb], tm[rb]);
      l_part[rb] = 0.f;
      t_max[rb] = -INFINITY;
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) O[cb][i] = 0.f;
    __syncthreads();   // the maxima are read before red is written again
    load_idx(k0);
    issue_tile(k0, buf0);
    load_idx(k0 + BN);
  }

  // ---- epilogue: row sums, partial results ---------------------------------
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();   // every wave is done with the tile buffers and red
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const float s = group_sum(l_part[rb]);
    if (lg == 0) red(16 * rb + l16)[w] = s;
  }
  {
    // lane holds row l32, columns col0 + 32 cb + 8 q + 4 half + (0..3)
    const int col0 = w * CPW;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint8_t* dst = buf0 + l32 * SROW + (col0 + 32 * cb + 8 * q + 4 * half) * 2;
        const f32x16& o = O[cb];
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
    for (int rb = 0; rb < NRB; ++rb) {
      const int row = 16 * rb + l16;
      if (row < nrows) {
        const f32x4 s4 = *reinterpret_cast<const f32x4*>(red(row));
        *reinterpret_cast<f32x2*>(p.ws_ml + (gro + idx0 + row) * 2) = f32x2{m_ref[rb], (s4[0] + s4[1]) + (s4[2] + s4[3])};
      }
    }
  }
  {
    constexpr int V16 = DV * 2 / 16;
    constexpr int NST = BM * V16 / 256;
    uint8_t* wso = reinterpret_cast<uint8_t*>(p.ws_o);
    u32x4 v[NST];
#pragma unroll
    for (int j = 0; j < NST; ++j) {
      const int e = tid + 256 * j;
      v[j] = *reinterpret_cast<const u32x4*>(buf0 + (e / V16) * SROW + 16 * (e % V16));
    }
#pragma unroll
    for (int j = 0; j < NST; ++j) {
      const int e = tid + 256 * j;
      const int row = e / V16;
      if (row < nrows)   // streaming stores: the partials are read once, by the merge
        __builtin_nontemporal_store(v[j], reinterpret_cast<u32x4*>(wso + ((gro + idx0 + row) * DV) * 2 + 16 * (e % V16)));
    }
  }
}

// ---------------------------------------------------------------------------
// The bf16 split with specialised waves, two per SIMD.  Waves 0..3 score:
// wave (kw, rw) takes 16 of a 32-position tile's keys (16 kw ..) against 32 of
// the query rows (32 rw ..), query block in registers, and writes P; waves 4..7
// form O^T for latent columns 128 (w - 4) .. + 127 of all 64 rows from the
// previous tile's P.  Phase k of a split scores tile k, runs PV of tile k - 1
// and copies tile k + 1, so the scoring and PV work of a phase overlap and each
// phase ends with one barrier; each SIMD holds one scoring and one PV wave, so
// it interleaves the two instruction streams (a single wave issues at most one
// instruction every four cycles).  LDS: three latent tile buffers (tile k is
// scored in phase k, multiplied in phase k + 1, and its buffer refilled with
// tile k + 3 in phase k + 2), two rope-key buffers and two P buffers (each read
// in one phase only), the rope part of the query block.  The PV waves copy the
// next tile (direct global -> LDS loads issued as inline asm, which the
// compiler does not track, all of them behind the phase's first MFMAs, so that
// they land while the rest of the PV runs) and wait for their copies (vmcnt)
// before the barrier that ends the phase; the scoring waves fetch the
// split's cache lines into L2 ahead of the copies (one load instruction a
// phase) and never wait for those loads inside the tile loop, so the fetches
// run many phases ahead.
// ---------------------------------------------------------------------------
template <int DR, bool SEL>
__global__ __launch_bounds__(512, 1) void absorbed_split_kernel(SplitArgs p) {
  constexpr int DA = 512, DV = 512;
  constexpr int BM = 64, BN = 32;
  constexpr int KL = DA / 32;             // 32-wide k steps of the score MFMA over the latent part
  constexpr int KR = DR / 32;             // ... over the rope part
  // Latent LDS rows: 1088 bytes (64 mod 256) with the 16-byte chunk index of row r
  // XOR-ed with lsw(r) = 2 ((r >> 2) & 1).  A ds_read_b128 serves 16 lanes per cycle
  // (lanes of one half-wave whose bits 2 ^ 3 ^ 4 agree), a ds_read_b64_tr_b16 32
  // lanes; with this layout the 16 lanes of a score fragment read (16 rows x 4
  // chunks) and the 32 lanes of a transposed V read (4 rows x 64 bytes) each touch
  // every bank once.  The copies apply the swizzle: lane i of a row's 1 KB copy
  // loads chunk i ^ lsw(r).
  constexpr int LRB = DA * 2 + 64;
  constexpr int RCH = DR / 8;             // 16-byte rope chunks per row
  constexpr int RRB = RCH * 16;           // rope LDS row: chunk c of row r stored at c ^ (r & 7)
  constexpr int BUF = BN * LRB;
  constexpr int RBUF = DR > 0 ? BN * RRB : 16;
  constexpr int QRBUF = DR > 0 ? BM * RRB : 16;
  constexpr int PRB = BN * 2 + 16;        // P row: 32 keys + pad (80 bytes: conflict-free reads and writes)
  constexpr int PBUF = BM * PRB;
  constexpr int CPW = DV / 4;             // latent columns per PV wave
  constexpr int NCB = CPW / 32;           // 32-column MFMA blocks per PV wave
  constexpr int SROW = DA * 2 + 48;       // epilogue staging row (unswizzled)
  static_assert(DR == 0 || (DR == 64 && BN * RCH == 4 * kWave), "rope width 0 or 64: one rope copy per wave");
  static_assert(BM * SROW <= 3 * BUF, "O staging fits in the tile buffers");

  __shared__ __attribute__((aligned(1024))) uint8_t lat[3 * BUF];
  __shared__ __attribute__((aligned(16))) uint8_t krope[2 * RBUF];
  __shared__ __attribute__((aligned(16))) uint8_t qrope[QRBUF];
  __shared__ __attribute__((aligned(16))) uint8_t pl[2 * PBUF];
  __shared__ __attribute__((aligned(16))) float red[BM * 2];   // per row: one float per key half
  __shared__ float mref[BM];                                   // per row: the softmax reference
  __shared__ uint32_t pfd[kWave];                              // landing slot of the L2 prefetch (never read)

  const int tid = threadIdx.x, lane = tid & 63;
  const int l16 = lane & 15, lg = lane >> 4;          // score layout: row block lane, key group
  const int half = lane >> 5, l32 = lane & 31;        // PV layout
  const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int T = (k1 - k0 + BN - 1) / BN;   // tiles of the split
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
    int lo = 0, hi = Kv;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (p.sel[sel0 + mid] < bound) lo = mid + 1; else hi = mid;
    }
    return lo;
  };
  // SEL: cache positions of the keys of the tile being copied (lane j: key j)
  // and of the one after it
  int sidx = 0, sidx_next = 0;
  auto load_idx = [&](int t0) {
    if (SEL) sidx_next = min(max(p.sel[sel0 + min(t0 + lane, k1 - 1)], 0), Kt - 1);
  };
  const int idx0 = rt * BM;
  const int nrows = min(BM, p.rows - idx0);
  const uint16_t* lbase = uniform_ptr(p.c_kv + p0 * DA);
  const uint16_t* rseq = p.k_pe + p0 * DR;

  // ---- tile copies, by the PV waves (cw = 0..3): NCP load instructions each ----
  // item j < NRC: rope block cw (rows 8 cw .. + 7; lane l fills row 8 cw + l / 8,
  // stored chunk l % 8, so it loads logical chunk (l % 8) ^ (l / 8)); the rest:
  // latent row cw + 4 (j - NRC), one 1 KB row per instruction.
  constexpr int NRC = DR > 0 ? 1 : 0;
  constexpr int NCP = NRC + BN / 4;
  const int rsw = (lane & 7) ^ (lane >> 3);
  const uint32_t lat_a = lds_addr(lat), krope_a = lds_addr(krope), qrope_a = lds_addr(qrope), pfd_a = lds_addr(pfd);
  // nb: the latent buffer (0..2), rb: the rope buffer (0, 1)
  const int cw = wu - 4;
  auto lsw = [](int r) { return ((r >> 2) & 1) << 1; };   // chunk swizzle of latent row r
  auto copy_item = [&](int t0, int nb, int rb, int j) {
    if (j < NRC) {
      const int blk = cw;
      const int key = 8 * blk + (lane >> 3);
      const int kr = SEL ? __shfl(sidx, key, kWave) : min(t0 + key, k1 - 1);
      dma_to<16>(rseq + (long long)kr * DR + 8 * rsw, krope_a + rb * RBUF + 1024 * blk);
    } else {
      const int key = cw + 4 * (j - NRC);
      const int kr = SEL ? __builtin_amdgcn_readlane(sidx, key) : __builtin_amdgcn_readfirstlane(min(t0 + key, k1 - 1));
      dma_sv_to<16>(lbase + (long long)kr * DA, (uint32_t)(16 * (lane ^ lsw(key))), lat_a + nb * BUF + key * LRB);
    }
  };
  auto issue_tile = [&](int t0, int nb, int rb) {
#pragma unroll
    for (int j = 0; j < NCP; ++j) copy_item(t0, nb, rb, j);
  };
  // Cache lines of positions [ta, tb) of the split -> L2 ahead of their copy:
  // this workgroup takes the positions p with (p - k0) % row_tiles == rt (the
  // row tiles of a split run on one XCD and share its L2), one 4-byte load per
  // 128-byte line (line e of the list for lane e; lanes past the list repeat
  // its last line), one load instruction per call.
  constexpr int LPP = DA / 64 + (DR > 0 ? 1 : 0);   // 128-byte lines per position
  auto prefetch_lines = [&](int ta, int tb, int e) {
    tb = min(tb, k1);
    const int rel = ta - k0;
    const int first = ta + ((rt - rel % p.row_tiles) + p.row_tiles) % p.row_tiles;
    const int cnt = first < tb ? (tb - 1 - first) / p.row_tiles + 1 : 0;
    const int nl = cnt * LPP;
    long long pos = p0 + k0;
    int ln = 0;
    if (nl > 0) {
      const int ee = min(e, nl - 1);
      const int j = ee / LPP;
      ln = ee - j * LPP;
      pos = p0 + first + (long long)p.row_tiles * j;
    }
    const uint16_t* src = ln < DA / 64 ? p.c_kv + pos * DA + 64 * ln : p.k_pe + pos * DR;
    dma_to<4>(src, pfd_a);
  };
  // The same for tile k + kPfAhead + 1 in phase k (positions [ta, ta + BN)),
  // with the per-phase arithmetic kept small (it runs on the scoring waves, whose
  // instruction count bounds the phase): the list starts at ta + pf_off, pf_off
  // stepping down by BN mod row_tiles a phase; this lane's entry (j, line) is fixed;
  // the one division by row_tiles uses a reciprocal (exact: the dividend is < BN).
  // With no list (tiles past the split) the load goes to the split's first line:
  // a build that skipped it measured slower (0.6 us per launch at 128 heads x 8
  // rows x 8192 positions, where every phase is such a phase).
  const int kPfAhead = p.pf_ahead;   // tiles of BN positions
  const int R = p.row_tiles;
  const int bn_mod = BN % R;
  int pf_off = ((rt - ((kPfAhead + 1) * BN) % R) % R + R) % R;
  const uint32_t rinv = R > 1 ? 0xffffffffu / (uint32_t)R + 1u : 0u;   // ceil(2^32 / R)
  const int lj = tid / LPP, lln = tid - lj * LPP;
  auto phase_prefetch = [&](int t0) {
    const int ta = t0 + (kPfAhead + 1) * BN;
    const int tb = min(ta + BN, k1);
    const int first = ta + pf_off;
    pf_off -= bn_mod;
    if (pf_off < 0) pf_off += R;
    long long pos = p0 + k0;   // no list: the split's first line again
    int ln = 0;
    if (first < tb) {
      const uint32_t x = (uint32_t)(tb - 1 - first);
      const int nl = ((R > 1 ? (int)__umulhi(x, rinv) : (int)x) + 1) * LPP;
      int j = lj;
      ln = lln;
      if (tid >= nl) {   // lanes past the list repeat its last line
        j = (nl - 1) / LPP;
        ln = (nl - 1) - j * LPP;
      }
      pos = p0 + first + (long long)R * j;
    }
    const uint16_t* src = ln < DA / 64 ? p.c_kv + pos * DA + 64 * ln : p.k_pe + pos * DR;
    dma_to<4>(src, pfd_a);
  };
  auto lgkm_barrier = [&]() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
  auto full_barrier = [&]() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
  const bool prefetch = !SEL;

  const long long qflat0 = (long long)b * p.rows + idx0;

  const long long gro = (long long)g * p.rows;
  if (wu < 4) {
    // ======================= scoring waves ====================================
    const int kw = wu & 1, rw = wu >> 1;   // keys 16 kw .., rows 32 rw ..
    const int srow = 32 * rw + l16;       // + 16 rb: this lane's rows
    // the query block's latent part -> the staging rows (tile buffers 1 and 2,
    // idle until the copy of tile 1), one 1 KB row per instruction (rows past
    // the last query row repeat it; their results are never stored)
    static_assert(BM * LRB <= 2 * BUF, "query staging fits in two tile buffers");
#pragma unroll
    for (int x = 0; x < BM / 4; ++x) {
      const int row = wu + 4 * x;
      dma_to<16>(p.q_lat + (qflat0 + min(row, nrows - 1)) * DA + 8 * (lane ^ lsw(row)), lat_a + BUF + row * LRB);
    }
    int kend[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) kend[rb] = min(k1, visible((idx0 + min(srow + 16 * rb, nrows - 1)) / p.H));
    const int kfull = __builtin_amdgcn_readfirstlane(min(k1, visible(idx0 / p.H)));   // every row sees these
    full_barrier();   // the query block, tile 0 (copied by the PV waves) in LDS
    // query block, latent part, from its staging rows into registers in the B
    // layout of the 16x16x32 MFMA: lane l holds row 32 rw + 16 rb + l % 16, k =
    // 32 ks + 8 (l / 16) ..; kept in accumulation registers (the MFMA reads its
    // B operand from there)
    u32x4 qf[2][KL];
    {
      const uint8_t* qsrc = lat + BUF + srow * LRB + 16 * (lg ^ lsw(srow));   // rows srow + 16 rb: the same swizzle
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int ks = 0; ks < KL; ++ks) {
          qf[rb][ks] = *reinterpret_cast<const u32x4*>(qsrc + 16 * rb * LRB + 64 * ks);
          asm("" : "+a"(qf[rb][ks]));
        }
    }
    // ... and its rope part (vector registers)
    auto rope_off = [&](int ks) { return 16 * ((4 * ks + lg) ^ (l16 & 7)); };
    const int qr_off = srow * RRB;                                         // + 16 rb RRB
    u32x4 qr[2][KR > 0 ? KR : 1];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int ks = 0; ks < KR; ++ks) qr[rb][ks] = *reinterpret_cast<const u32x4*>(qrope + qr_off + 16 * rb * RRB + rope_off(ks));
    lgkm_barrier();   // the staging rows are free for tile 1
    // the split's first lines -> L2 (tiles 1 .. kPfAhead); not waited for
    if (prefetch) {
      const int ta = k0 + BN, tb = min(k1, k0 + (kPfAhead + 1) * BN);
      const int first = ta + ((rt - BN % p.row_tiles) + p.row_tiles) % p.row_tiles;
      const int nl = (first < tb ? (tb - 1 - first) / p.row_tiles + 1 : 0) * LPP;
      for (int e0 = 0; e0 < nl; e0 += 256) prefetch_lines(ta, tb, e0 + tid);
    }

    float m_ref[2], l_part[2], t_max[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) { m_ref[rb] = -INFINITY; l_part[rb] = 0.f; t_max[rb] = -INFINITY; }
    bool rerun = false;
    const int kq_off = (16 * kw + l16) * LRB + 16 * (lg ^ lsw(l16));      // + 64 ks
    const int kr_off = (16 * kw + l16) * RRB;
    const int pw_off = srow * PRB + (16 * kw + 4 * lg) * 2;                // + 16 rb PRB
    for (;;) {
      const uint8_t* cur = lat;           // tile k's buffer
      int nb = 1;                         // tile k + 1's (0..2)
      for (int k = 0; k <= T; ++k) {
        const int t0 = k0 + k * BN;
        // the cache lines of tile k + kPfAhead + 1 (a quarter of them per wave)
        if (prefetch && !rerun) phase_prefetch(t0);
        if (k < T) {
          const uint8_t* kro = krope + (k & 1) * RBUF;
          // ---- scores: S^T [16 keys x 32 rows] ---------------------------------
          f32x4 acc[2];
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
          {
            // k steps 0 .. KL - 1 over the latent part, then KR over the rope
            // part, key fragments read PF steps ahead of their MFMAs
            constexpr int PF = 4, NK = KL + KR;
            const uint8_t* kq = cur + kq_off;
            auto kfrag = [&](int ks) -> u32x4 {
              return ks < KL ? *reinterpret_cast<const u32x4*>(kq + 64 * ks)
                             : *reinterpret_cast<const u32x4*>(kro + kr_off + rope_off(ks - KL));
            };
            u32x4 ka[PF];
#pragma unroll
            for (int c = 0; c < PF; ++c) ka[c] = kfrag(c);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < NK; ++ks) {
              const u32x4 a = ka[ks % PF];
              if (ks + PF < NK) ka[ks % PF] = kfrag(ks + PF);
#pragma unroll
              for (int rb = 0; rb < 2; ++rb) acc[rb] = mfma16(a, ks < KL ? qf[rb][ks] : qr[rb][ks - KL], acc[rb]);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          // acc[rb][i] = q . k for key t0 + 16 kw + 4 lg + i, row srow + 16 rb
          if (t0 + BN > kfull) {   // a tile past some row's causal end (uniform branch)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (t0 + 16 * kw + 4 * lg + i >= kend[rb]) acc[rb][i] = -INFINITY;
          }
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            t_max[rb] = fmaxf(fmaxf(t_max[rb], fmaxf(acc[rb][0], acc[rb][1])), fmaxf(acc[rb][2], acc[rb][3]));
          // the split's first tile sets each row's reference (a row sees a
          // prefix of the split's positions, so its first finite scores are here)
          if (k == 0 && !rerun) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
              const float mx = group_max(fmaxf(fmaxf(acc[rb][0], acc[rb][1]), fmaxf(acc[rb][2], acc[rb][3])));
              if (lg == 0) red[(srow + 16 * rb) * 2 + kw] = mx * p.sl2;
            }
            lgkm_barrier();   // (the PV waves meet it at the same point of phase 0)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
              const f32x2 r2 = *reinterpret_cast<const f32x2*>(&red[(srow + 16 * rb) * 2]);
              m_ref[rb] = fmaxf(r2[0], r2[1]);
              if (kw == 0 && lg == 0) mref[srow + 16 * rb] = m_ref[rb];
            }
          }
          // P = 2^(s - m) in bf16 (rows without a finite reference use 0: their
          // masked keys give 0); the row sums add the rounded weights PV uses
          uint8_t* pw = pl + (k & 1) * PBUF + pw_off;
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            const float mb = m_ref[rb] == -INFINITY ? 0.f : m_ref[rb];
            float e[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) e[i] = __builtin_amdgcn_exp2f(fmaf(acc[rb][i], p.sl2, -mb));
            u32x2 v;
            v[0] = pack_bf16(e[0], e[1]);
            v[1] = pack_bf16(e[2], e[3]);
            *reinterpret_cast<u32x2*>(pw + 16 * rb * PRB) = v;
            l_part[rb] = add_bf16x2(v[1], add_bf16x2(v[0], l_part[rb]));
          }
        }
        lgkm_barrier();   // P(k) written
        cur = lat + nb * BUF;
        nb = nb == 2 ? 0 : nb + 1;
      }
      // Did some row's scores exceed its reference by more than 2^kRefSlack?
      // Then its P, O and l may have overflowed: raise every reference to the
      // row's maximum over the whole split and run the split again (the second
      // pass cannot trigger another: its references bound every score).
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const float mx = group_max(t_max[rb]);
        if (lg == 0) red[(srow + 16 * rb) * 2 + kw] = mx * p.sl2;
      }
      lgkm_barrier();
      const f32x2 rl = *reinterpret_cast<const f32x2*>(&red[lane * 2]);
      const float mr = mref[lane];
      const bool over = mr != -INFINITY && fmaxf(rl[0], rl[1]) > mr + kRefSlack;
      if (rerun || __ballot(over) == 0) break;
      rerun = true;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const f32x2 r2 = *reinterpret_cast<const f32x2*>(&red[(srow + 16 * rb) * 2]);
        m_ref[rb] = m_ref[rb] == -INFINITY ? m_ref[rb] : fmaxf(m_ref[rb], fmaxf(r2[0], r2[1]));
        l_part[rb] = 0.f;
        t_max[rb] = -INFINITY;
      }
      lgkm_barrier();   // red read by every wave before the next write
      lgkm_barrier();   // the PV waves copy tile 0 again
    }
    // ---- epilogue: row sums; the PV waves stage O -----------------------------
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no prefetch load outlives the workgroup
    lgkm_barrier();   // every wave is done reading red
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const float s = group_sum(l_part[rb]);
      if (lg == 0) red[(srow + 16 * rb) * 2 + kw] = s;
    }
    lgkm_barrier();   // row sums and the staged O visible
    if (kw == 0 && lg == 0) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int row = srow + 16 * rb;
        if (row < nrows) {
          const f32x2 s2 = *reinterpret_cast<const f32x2*>(&red[row * 2]);
          *reinterpret_cast<f32x2*>(p.ws_ml + (gro + idx0 + row) * 2) = f32x2{m_ref[rb], s2[0] + s2[1]};
        }
      }
    }
  } else {
    // ======================= PV waves =========================================
    // prologue: tile 0 and the query block's rope part (same swizzled layout as
    // the rope keys: 64 rows, two copies per wave) -> LDS
    load_idx(k0);
    sidx = sidx_next;
    issue_tile(k0, 0, 0);
    load_idx(k0 + BN);
    if (DR > 0) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int j = cw + 4 * x;
        const int row = 8 * j + (lane >> 3);
        dma_to<16>(p.q_pe + (qflat0 + min(row, nrows - 1)) * DR + 8 * rsw, qrope_a + 1024 * j);
      }
    }
    f32x16 O[2][NCB];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) O[rb][cb][i] = 0.f;
    full_barrier();   // tile 0, rope queries in LDS
    lgkm_barrier();   // the scoring waves have read the query block
    const int G = lane >> 4, s16 = lane & 15;
    // rows 16 kc + 4 ld + 8 (G >> 1) + s16 / 4: bit 2 of the row is ld, so the rows
    // of the ld = 1 reads have chunk bit 1 (byte bit 5, i.e. G & 1) flipped
    const int tr_col = (cw * CPW + 16 * (G & 1) + 4 * (s16 & 3)) * 2;
    const int tr_off = (8 * (G >> 1) + (s16 >> 2)) * LRB + tr_col;
    const int tr_off1 = (8 * (G >> 1) + (s16 >> 2)) * LRB + (tr_col ^ 32);
    const int pa_off = l32 * PRB + 16 * half;                              // + rb*32*PRB + 32 kc
    bool rerun = false;
    for (;;) {
      uint8_t* prv = lat + 2 * BUF;       // tile k - 1's buffer
      int nb = 1;                         // tile k + 1's (0..2)
      for (int k = 0; k <= T; ++k) {
        const int t0 = k0 + k * BN;
        sidx = sidx_next;          // positions of tile k + 1
        load_idx(t0 + 2 * BN);     // ... and of tile k + 2
        const bool cp = k + 1 < T;
        const int rnx = (k + 1) & 1;
        if (k == 0 && cp) issue_tile(t0 + BN, nb, rnx);   // no PV in phase 0
        if (k == 0 && !rerun) lgkm_barrier();   // the scoring waves' exchange of the references
        if (k > 0) {
          // ---- PV: O^T [128 columns x 64 rows] += V^T P^T for tile k - 1 ---------
          const uint8_t* pa = pl + ((k - 1) & 1) * PBUF + pa_off;
          const uint8_t* vb = prv + tr_off;
          const uint8_t* vb1 = prv + tr_off1;
          auto vfrag = [&](int kc, int cb) {
            u32x4 bv;
#pragma unroll
            for (int ld = 0; ld < 2; ++ld) {
              const uint8_t* src = (ld ? vb1 : vb) + (16 * kc + 4 * ld) * LRB + 64 * cb;
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
            // the copy of tile k + 1, all of it behind the first MFMAs: it then
            // lands while the rest of the PV runs, not after it
            if (cp && st == 0) {
#pragma unroll
              for (int j = 0; j < NCP; ++j) copy_item(t0 + BN, nb, rnx, j);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        full_barrier();   // this wave's copies have landed; P(k - 1) consumed
        prv = prv + BUF == lat + 3 * BUF ? lat : prv + BUF;
        nb = nb == 2 ? 0 : nb + 1;
      }
      // the decision of the scoring waves, from the same values
      lgkm_barrier();
      const f32x2 rl = *reinterpret_cast<const f32x2*>(&red[lane * 2]);
      const float mr = mref[lane];
      const bool over = mr != -INFINITY && fmaxf(rl[0], rl[1]) > mr + kRefSlack;
      if (rerun || __ballot(over) == 0) break;
      rerun = true;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int i = 0; i < 16; ++i) O[rb][cb][i] = 0.f;
      lgkm_barrier();
      load_idx(k0);
      sidx = sidx_next;
      issue_tile(k0, 0, 0);
      load_idx(k0 + BN);
      full_barrier();
    }
    // ---- epilogue: O -> bf16 staging rows (the tile buffers are free) ----------
    lgkm_barrier();   // every wave is done reading red
    {
      // lane holds row 32 rb + l32, columns col0 + 32 cb + 8 q + 4 half + (0..3)
      const int col0 = cw * CPW;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint8_t* dst = lat + (32 * rb + l32) * SROW + (col0 + 32 * cb + 8 * q + 4 * half) * 2;
            const f32x16& o = O[rb][cb];
            u32x2 v;
            v[0] = pack_bf16(o[4 * q], o[4 * q + 1]);
            v[1] = pack_bf16(o[4 * q + 2], o[4 * q + 3]);
            *reinterpret_cast<u32x2*>(dst) = v;
          }
    }
    lgkm_barrier();   // row sums and the staged O visible
  }
  // ---- every wave: the staged rows out with 16-byte stores ---------------------
  {
    constexpr int V16 = DV * 2 / 16;                // 16-byte chunks per row
    constexpr int NST = BM * V16 / 512;
    uint8_t* wso = reinterpret_cast<uint8_t*>(p.ws_o);
    u32x4 v[NST];
#pragma unroll
    for (int j = 0; j < NST; ++j) {
      const int e = tid + 512 * j;
      v[j] = *reinterpret_cast<const u32x4*>(lat + (e / V16) * SROW + 16 * (e % V16));
    }
#pragma unroll
    for (int j = 0; j < NST; ++j) {
      const int e = tid + 512 * j;
      const int row = e / V16;
      if (row < nrows)   // streaming stores: the partials are read once, by the merge
        __builtin_nontemporal_store(v[j], reinterpret_cast<u32x4*>(wso + ((gro + idx0 + row) * DV) * 2 + 16 * (e % V16)));
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
namespace {
SplitArgs split_args(const AbsorbedLaunch& q) {
  SplitArgs a{};
  a.q_lat = (const uint16_t*)q.q_lat; a.q_pe = (const uint16_t*)q.q_pe; a.q8 = (const uint8_t*)q.q8;
  a.c_kv = (const uint16_t*)q.c_kv; a.k_pe = (const uint16_t*)q.k_pe;
  a.off = q.off_dev; a.off0 = q.off0; a.kv1 = q.kv1;
  a.ws_o = (uint16_t*)q.ws_o; a.ws_ml = q.ws_ml;
  a.B = q.B; a.L = q.L; a.H = q.H; a.rows = q.L * q.H;
  a.row_tiles = q.plan.row_tiles; a.chunk = q.plan.chunk; a.n_items = q.plan.n_items;
  a.sl2 = q.scale * 1.4426950408889634f;
  // L2 prefetch window of the bf16 kernel: an XCD's 32 CUs run 32 / row_tiles
  // distinct splits at a time, each with pf_ahead tiles (36 KB) in flight;
  // about 2 row_tiles tiles keeps that near 2 MB of its 4 MB L2
  a.pf_ahead = std::min(32, std::max(4, 2 * a.row_tiles));
  return a;
}
unsigned grid_of(int n_items) { return (unsigned)(((n_items + kXcds - 1) / kXcds) * kXcds); }
}  // namespace

hipError_t absorbed_attn_bf16(const AbsorbedLaunch& q, hipStream_t st) {
  const SplitArgs a = split_args(q);
  if (q.r != 512) return hipErrorInvalidValue;
  const dim3 grid(grid_of(a.n_items));
  switch (q.rope) {
    case 0:  hipLaunchKernelGGL((absorbed_split_kernel<0, false>), grid, dim3(512), 0, st, a); break;
    case 64: hipLaunchKernelGGL((absorbed_split_kernel<64, false>), grid, dim3(512), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The fp8 kernel takes 32 query rows per workgroup (two workgroups per CU), the
// plan's splits with twice its 64-row tiles.
void f8_rows(SplitArgs& a, int rope) {
  a.row_tiles = (a.rows + 31) / 32;
  a.n_items = (a.n_items / ((a.rows + 63) / 64)) * a.row_tiles;
  a.pf_ahead = std::min(16, std::max(2, a.row_tiles / 2));
  const int lines = (64 * (512 + rope) + 127) / 128 + 2;   // a tile's code lines and its scales' lines
  a.pf_lines = std::min(256, (lines + a.row_tiles - 1) / a.row_tiles);
}

hipError_t absorbed_attn_fp8(const AbsorbedLaunch& q, const void* codes, const float* scales, hipStream_t st) {
  SplitArgs a = split_args(q);
  a.c8 = (const uint8_t*)codes; a.s8 = scales;
  f8_rows(a, q.rope);
  if (q.r != 512) return hipErrorInvalidValue;
  const dim3 grid(grid_of(a.n_items));
  const bool q8 = a.q8 != nullptr;
  switch (q.rope) {
    case 0:
      if (q8) hipLaunchKernelGGL((absorbed_split_f8_kernel<0, false, true>), grid, dim3(256), 0, st, a);
      else hipLaunchKernelGGL((absorbed_split_f8_kernel<0, false, false>), grid, dim3(256), 0, st, a);
      break;
    case 64:
      if (q8) hipLaunchKernelGGL((absorbed_split_f8_kernel<64, false, true>), grid, dim3(256), 0, st, a);
      else hipLaunchKernelGGL((absorbed_split_f8_kernel<64, false, false>), grid, dim3(256), 0, st, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t absorbed_attn_sparse_fp8(const AbsorbedLaunch& q, const void* codes, const float* scales,
                                    const int32_t* sel, const int32_t* koff_dev, int koff0, int kvt1, hipStream_t st) {
  SplitArgs a = split_args(q);
  a.c8 = (const uint8_t*)codes; a.s8 = scales;
  a.sel = sel; a.koff = koff_dev; a.koff0 = koff0; a.kvt1 = kvt1;
  f8_rows(a, q.rope);
  if (q.r != 512) return hipErrorInvalidValue;
  const dim3 grid(grid_of(a.n_items));
  switch (q.rope) {
    case 0:  hipLaunchKernelGGL((absorbed_split_f8_kernel<0, true, false>), grid, dim3(256), 0, st, a); break;
    case 64: hipLaunchKernelGGL((absorbed_split_f8_kernel<64, true, false>), grid, dim3(256), 0, st, a); break;
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
    case 0:  hipLaunchKernelGGL((absorbed_split_kernel<0, true>), grid, dim3(512), 0, st, a); break;
    case 64: hipLaunchKernelGGL((absorbed_split_kernel<64, true>), grid, dim3(512), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
