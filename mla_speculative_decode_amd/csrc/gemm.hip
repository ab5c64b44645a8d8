// gemm.hip -- the two dense contractions around the attention kernels:
//
//   fold    q_lat[m, h, :] = q_nope[m, h, :] . W_UK[h]          (absorbed route)
//   expand  K[t, h, :n] = W_UK[h] . c_kv[t],  K[t, h, n:] = k_pe[t],
//           V[t, h, :]  = c_kv[t] . W_UV[h]                      (materialised route)
//
// ("One guard, 110x off the verify step", section "The defect": fold the
// up-projection into the query; expand the cached latent into full K and V.)
//
// bf16 uses MFMA with fp32 accumulation.  MFMA operands need the contraction
// index contiguous per lane; W_UK [H, n, r] (fold contracts over n) and W_UV
// [H, r, v] (the expand contracts over r) store it strided: both the fold's
// small-M GEMM and the expand read those fragments transposed from LDS
// (ds_read_b64_tr_b16).  The fold is a small-M product (M = B*L rows per head): each
// workgroup reads its weight tile once for up to 64 rows, the weight stream
// being the cost.  float32 uses plain VALU loops.

#include "mla_device.h"
#include "internal.h"

namespace mla {

// ---------------------------------------------------------------------------
// Small-M batched GEMM per head, bf16 MFMA:  C[h][m, :] = A[h][m, :] . W[h]
// with W[h] row-major [K x N] (N contiguous), A and C bf16, fp32 accumulation.
// Used for the fold (A = q_nope, W = W_UK[h], C = q_lat).  Workgroup = (head,
// 64 output columns, MT rows): the W tile [K x 64] and the A tile are loaded
// into registers with 16-byte loads, written to LDS (padded rows), and
// multiplied with 16x16x32 MFMAs, W fragments read transposed from the
// row-major tile (ds_read_b64_tr_b16).  Each wave owns 16 output columns; the
// weight stream is read once per MT rows.
// ---------------------------------------------------------------------------
//
// Q8 (the fold for the fp8 route): the rows are also written as the E4M3 query
// block (the layout of kQ8TileBytes): each 32-wide block of an output row is
// columns 32 jb .. + 31 of a tile; the tile goes through LDS and one thread
// quantises each (row, block).  The codes are those of the bf16-rounded
// products (the values q_lat holds).  The rope part (q_pe) is spread over the
// same workgroups, one thread per (row, 32-wide block).
template <int MT, int KMAX, bool Q8>
__global__ __launch_bounds__(256) void gemm_smallm_kernel(GemmArgs g) {
  constexpr int WRB = 64 * 2 + 16;          // W row: 64 bf16 + pad
  constexpr int ARB = KMAX * 2 + 16;        // A row: K bf16 + pad
  constexpr int RB = MT / 16;
  __shared__ __attribute__((aligned(16))) uint8_t wt[KMAX * WRB];
  __shared__ __attribute__((aligned(16))) uint8_t at[MT * ARB];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int item = xcd_item(blockIdx.x, g.n_items);
  if (item >= g.n_items) return;

  const int CT = g.N / 64, MTS = (g.M + MT - 1) / MT;
  const int mt = item % MTS;
  const int tmp = item / MTS;
  const int ct = tmp % CT, h = tmp / CT;
  const int K = g.K, m0 = mt * MT;

  // ---- Q8: rope part of the query block, spread over the GEMM's workgroups:
  // thread tid takes block u = tid * items + item of the rows' rope parts (row
  // b L H + l H + h, 32-wide block j); its loads go out first and it is
  // quantised as soon as they land, while the tiles' loads are in flight
  u32x4 rv[4];
  long long rrow = 0;
  int rj = 0;
  bool has_rope = false;
  if (Q8 && g.rope > 0) {
    const int NBR = g.rope / 32;
    const long long u = (long long)tid * g.n_items + item;
    if (u < (long long)g.M * g.H * NBR) {
      has_rope = true;
      rrow = u / NBR;
      rj = (int)(u - rrow * NBR);
#pragma unroll
      for (int c = 0; c < 4; ++c) rv[c] = ld16(g.q_pe + rrow * g.rope + 32 * rj + 8 * c);
    }
  }
  auto rope_block = [&]() {
    const int LH = g.L * g.H;
    const int b = (int)(rrow / LH), iseq = (int)(rrow - (long long)b * LH);
    const int r = iseq & 31;
    uint8_t* const tb = g.q8 + ((long long)b * g.row_tiles + (iseq >> 5)) * kQ8TileBytes;
    const int e = e4m3_scale_exponent_bf16(absmax32(rv));
    const float sc = __uint_as_float((uint32_t)(e + 127) << 23);
    const u32x2 c0 = e4m3x8(rv[0], sc), c1 = e4m3x8(rv[1], sc), c2 = e4m3x8(rv[2], sc), c3 = e4m3x8(rv[3], sc);
    uint8_t* const rp = tb + kQ8RopeOff + 16 * (kWave * (r >> 4) + 32 * rj + (r & 15));
    st16(rp, u32x4{c0[0], c0[1], c1[0], c1[1]});
    st16(rp + 16 * 16, u32x4{c2[0], c2[1], c3[0], c3[1]});
    uint32_t* const sp = reinterpret_cast<uint32_t*>(tb + kQ8ScaleOff) + kWave * (2 * (r >> 4) + 1) + (r & 15);
    sp[16 * rj] = (uint32_t)(e + 127);
    sp[16 * (rj + 2)] = 127u;
  };

  // ---- W tile: K rows x 64 columns (K * 8 chunks of 16 B) --------------------
  const uint16_t* wsrc = g.W + (long long)h * K * g.N + ct * 64;
  constexpr int WCH_T = KMAX * 8 / 256;     // chunks per thread at K = KMAX
  u32x4 wst[WCH_T];
#pragma unroll
  for (int x = 0; x < WCH_T; ++x) {
    const int C = tid + 256 * x;
    if (C < K * 8) wst[x] = ld16(wsrc + (long long)(C >> 3) * g.N + 8 * (C & 7));
  }
  // ---- A tile: MT rows x K (8 elements per 16-byte chunk) ----------------------
  constexpr int ACH_T = MT * KMAX / 8 / 256;
  u32x4 ast[ACH_T];
  const int KC = K / 8;                     // chunks per A row
#pragma unroll
  for (int x = 0; x < ACH_T; ++x) {
    const int C = tid + 256 * x;
    const int r = C / KC, c = C % KC;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (C < MT * KC && m0 + r < g.M)
      v = ld16(g.A + (long long)h * g.a_head + (long long)(m0 + r) * g.a_row + (long long)c * 8);
    ast[x] = v;
  }
  if (Q8 && has_rope) rope_block();   // waits for the rope loads only (issued first)
#pragma unroll
  for (int x = 0; x < WCH_T; ++x) {
    const int C = tid + 256 * x;
    if (C < K * 8) st16(wt + (C >> 3) * WRB + 16 * (C & 7), wst[x]);
  }
#pragma unroll
  for (int x = 0; x < ACH_T; ++x) {
    const int C = tid + 256 * x;
    const int r = C / KC, c = C % KC;
    if (C < MT * KC) st16(at + r * ARB + c * 16, ast[x]);
  }
  __syncthreads();

  // ---- MFMA: wave w -> columns 16w..16w+15 ------------------------------------
  const int r16 = lane & 15, G = lane >> 4;
  const uint8_t* wb = wt + (8 * G + (r16 >> 2)) * WRB + (16 * w + 4 * (r16 & 3)) * 2;
  f32x4 acc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nrb = min(RB, (g.M - m0 + 15) / 16);
  for (int ks = 0; ks < K / 32; ++ks) {
    u32x4 bv;
#pragma unroll
    for (int ld = 0; ld < 2; ++ld) {
      const v4i16 rr = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16*)(wb + (32 * ks + 4 * ld) * WRB));
      const u32x2 r2 = __builtin_bit_cast(u32x2, rr);
      bv[2 * ld] = r2[0];
      bv[2 * ld + 1] = r2[1];
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (rb < nrb) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(at + (16 * rb + r16) * ARB + (32 * ks + 8 * G) * 2);
        acc[rb] = mfma16(a, bv, acc[rb]);
      }
    }
  }
  // C layout: lane holds column 16w + lane%16, rows 4*(lane/16) + x
  if (!Q8 || g.C) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int m = m0 + 16 * rb + 4 * G + x;
        if (m < g.M) {
          const long long o = (long long)h * g.c_head + (long long)m * g.c_row + ct * 64 + 16 * w + r16;
          g.C[o] = __builtin_bit_cast(uint16_t, (__bf16)acc[rb][x]);
        }
      }
  }
  if (Q8) {
    // ---- latent part of the query block: the bf16-rounded tile -> LDS, then
    // one thread per (row, 32-column block): row m = b L + l is sequence row
    // l H + h; block jb of this tile is block 2 (ct % 2) + jb of step ct / 2,
    // half ct % 2 of lane groups 2 jb and 2 jb + 1
    // the staging reuses the A tile's LDS once every wave is past its MFMAs
    static_assert(MT * 64 * 2 <= MT * ARB, "output tile fits in the A tile");
    uint16_t* const stg = reinterpret_cast<uint16_t*>(at);
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int x = 0; x < 4; ++x) stg[(16 * rb + 4 * G + x) * 64 + 16 * w + r16] = __builtin_bit_cast(uint16_t, (__bf16)acc[rb][x]);
    __syncthreads();
    const int row_t = tid >> 1, jb = tid & 1, m = m0 + row_t;
    if (tid < 2 * MT && m < g.M) {
      u32x4 v[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = *reinterpret_cast<const u32x4*>(stg + row_t * 64 + 32 * jb + 8 * c);
      const int e = e4m3_scale_exponent_bf16(absmax32(v));
      const float sc = __uint_as_float((uint32_t)(e + 127) << 23);
      const u32x2 c0 = e4m3x8(v[0], sc), c1 = e4m3x8(v[1], sc), c2 = e4m3x8(v[2], sc), c3 = e4m3x8(v[3], sc);
      const int b = m / g.L, iseq = (m - b * g.L) * g.H + h, r = iseq & 31;
      const int ks = ct >> 1, hh = ct & 1;
      uint8_t* const tb = g.q8 + ((long long)b * g.row_tiles + (iseq >> 5)) * kQ8TileBytes;
      uint8_t* const cd = tb + 16 * ((2 * (4 * (r >> 4) + ks) + hh) * kWave + 32 * jb + (r & 15));
      st16(cd, u32x4{c0[0], c0[1], c1[0], c1[1]});
      st16(cd + 16 * 16, u32x4{c2[0], c2[1], c3[0], c3[1]});
      tb[kQ8ScaleOff + 4 * (kWave * 2 * (r >> 4) + 16 * (2 * hh + jb) + (r & 15)) + ks] = (uint8_t)(e + 127);
    }
  }
}

hipError_t gemm_smallm(const GemmArgs& a0, hipStream_t st) {
  GemmArgs a = a0;
  if (a.K % 32 != 0 || a.K > 512 || a.N % 64 != 0) return hipErrorInvalidValue;
  const bool q8 = a.q8 != nullptr;
  if (q8 && (a.N != 512 || !(a.rope == 0 || a.rope == 64) || a.L < 1 || a.M % a.L != 0)) return hipErrorInvalidValue;
  const int MT = a.M <= 16 ? 16 : 64;       // rows per workgroup
  a.n_items = a.H * (a.N / 64) * ((a.M + MT - 1) / MT);
  // Q8: the rope blocks (M H rope / 32) are spread over the workgroups' 256 threads
  if (q8 && (long long)a.M * a.H * (a.rope / 32) > 256LL * a.n_items) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)(((a.n_items + kXcds - 1) / kXcds) * kXcds);
  // LDS and staging registers are sized by KMAX: small K keeps several workgroups per CU
  const int KM = a.K <= 128 ? 128 : (a.K <= 256 ? 256 : 512);
#define MLA_GEMM(M_, KM_)                                                                                \
  if (MT == M_ && KM == KM_) {                                                                           \
    if (q8) hipLaunchKernelGGL((gemm_smallm_kernel<M_, KM_, true>), dim3(grid), dim3(256), 0, st, a);    \
    else hipLaunchKernelGGL((gemm_smallm_kernel<M_, KM_, false>), dim3(grid), dim3(256), 0, st, a);      \
    return hipGetLastError();                                                                            \
  }
  MLA_GEMM(16, 128) MLA_GEMM(64, 128) MLA_GEMM(16, 256) MLA_GEMM(64, 256) MLA_GEMM(16, 512) MLA_GEMM(64, 512)
#undef MLA_GEMM
  return hipErrorInvalidValue;
}

// the fold for the fp8 route: q_lat (optional) and the E4M3 query block of
// the sequence rows (latent part from the bf16 products, rope part from q_pe)
hipError_t fold_query_fp8(int B, int L, int H, int n, int rope, const void* q_nope, const void* w_uk,
                          const void* q_pe, void* q_lat, void* q8, hipStream_t st) {
  if (n % 32 != 0 || n > 512) return hipErrorInvalidValue;
  GemmArgs a{};
  a.A = (const uint16_t*)q_nope; a.a_row = (long long)H * n; a.a_head = n;
  a.W = (const uint16_t*)w_uk;
  a.C = (uint16_t*)q_lat; a.c_row = (long long)H * 512; a.c_head = 512;
  a.M = B * L; a.K = n; a.N = 512; a.H = H;
  a.q8 = (uint8_t*)q8; a.q_pe = (const uint16_t*)q_pe;
  a.L = L; a.rope = rope; a.row_tiles = (L * H + 31) / 32;
  return gemm_smallm(a, st);
}

__global__ __launch_bounds__(256) void fold_f32_kernel(const float* __restrict__ q_nope, const float* __restrict__ w_uk,
                                                       float* __restrict__ q_lat, long long total, int H, int n, int r) {
  for (long long o = blockIdx.x * 256LL + threadIdx.x; o < total; o += (long long)gridDim.x * 256) {
    const int c = (int)(o % r);
    const long long mh = o / r;
    const int h = (int)(mh % H);
    const float* q = q_nope + mh * n;
    const float* wk = w_uk + (long long)h * n * r + c;
    float a = 0.f;
    for (int j = 0; j < n; ++j) a = fmaf(q[j], wk[(long long)j * r], a);
    q_lat[o] = a;
  }
}

hipError_t fold_query(mla_dtype_t dt, int rows, int H, int n, int r, const void* q_nope, const void* w_uk,
                      void* q_lat, hipStream_t st) {
  if (dt == kBF16) {
    if (n % 32 != 0 || n > 512 || r % 64 != 0) return hipErrorInvalidValue;
    GemmArgs a{};
    a.A = (const uint16_t*)q_nope; a.a_row = (long long)H * n; a.a_head = n;
    a.W = (const uint16_t*)w_uk;
    a.C = (uint16_t*)q_lat; a.c_row = (long long)H * r; a.c_head = r;
    a.M = rows; a.K = n; a.N = r; a.H = H;
    return gemm_smallm(a, st);
  }
  const long long total = (long long)rows * H * r;
  const long long blocks = (total + 255) / 256;
  hipLaunchKernelGGL(fold_f32_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, st,
                     (const float*)q_nope, (const float*)w_uk, (float*)q_lat, total, H, n, r);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// expand, bf16: two plain GEMMs over the cached latent A = c_kv [T x r]
// (contraction over r, fp32 accumulation, bf16 results):
//   K part (NN = false): C[t, q] = sum_c A[t, c] W_UK[q, c] with W_UK viewed
//       as [(H n) x r], q = h n + j; C[t, q] is stored at K[t, q / n, q % n];
//   V part (NN = true):  C[t, q] = sum_c A[t, c] W_UV[q / v, c, q % v], and C
//       is V viewed as [T x (H v)].
// Workgroup tile 128 positions x 128 columns; k steps of 64, double-buffered
// in LDS and filled by direct-to-LDS loads (each wave instruction writes 1 KB,
// lane l at bytes 16l..16l+15).  Which global 16-byte chunk a lane fetches
// sets an XOR swizzle of the chunks inside an LDS row, so the fragment reads
// are free of bank conflicts without padding.  The product is computed
// transposed, C^T = B^T A^T, in 32x32x16 MFMAs (wave (wm, wn) owns 64 x 64),
// so a lane holds 4 consecutive output columns of one position; the tile is
// staged through LDS and leaves with 16-byte row-contiguous stores.  Items
// are ordered so that each XCD takes one contiguous range of column tiles for
// all row tiles: its weight tiles stay in its L2 while the latent rows pass.
// ---------------------------------------------------------------------------
struct ExpandArgs {
  const uint16_t* a;   // c_kv [T, r]
  const uint16_t* w;   // W_UK [H, n, r] (K part) or W_UV [H, r, v] (V part)
  uint16_t* out;       // K [T, H, n + rope] or V [T, H, v]
  long long T;
  int H, r, n, v, rope;
  int ncols;           // H n (K part) or H v (V part)
  int MT, NTX;         // row tiles; column tiles per XCD
  int n_items;         // kXcds * MT * NTX
};

template <bool NN>
__global__ __launch_bounds__(256, 2) void expand_gemm_kernel(ExpandArgs p) {
  constexpr int BM = 128, BN = 128, BK = 64;
  constexpr int ABYTES = BM * BK * 2;     // rows of 128 B (8 chunks)
  constexpr int BBYTES = BN * BK * 2;     // NT: rows of 128 B per column; NN: rows of 256 B per k
  constexpr int STAGE = ABYTES + BBYTES;
  constexpr int CP = BN * 2 + 16;         // staging row pitch of the output tile (bytes)
  static_assert(BM * CP <= 2 * STAGE, "output staging fits in the stage buffers");
  __shared__ __attribute__((aligned(1024))) uint8_t sm[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int item = __builtin_amdgcn_readfirstlane(xcd_item(blockIdx.x, p.n_items));
  if (item >= p.n_items) return;
  const int per = p.MT * p.NTX;
  const int xb = item / per, rem = item - xb * per;
  const int mt = rem / p.NTX;
  const int nt = __builtin_amdgcn_readfirstlane(xb * p.NTX + (rem - mt * p.NTX));
  if (nt * BN >= p.ncols) return;
  const long long t0 = (long long)mt * BM;
  const int q0 = nt * BN;
  typedef __attribute__((address_space(3))) void* lds_ptr;

  // per-lane source offsets (elements) that do not change with the k step
  long long a_src[4];
  long long b_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int x = w + 4 * i;                       // instruction slot: 1 KB of the tile
    const int row = 8 * x + (lane >> 3);           // A: 8 rows of 8 chunks per instruction
    const int c = (lane & 7) ^ (lane >> 3);        // logical chunk landing in physical slot lane & 7
    long long t = t0 + row;
    t = t < p.T ? t : p.T - 1;
    a_src[i] = t * p.r + 8 * c;
    if (!NN) {
      int q = q0 + row;                            // weight row = output column
      q = q < p.ncols ? q : p.ncols - 1;
      b_src[i] = (long long)q * p.r + 8 * c;
    } else {
      const int krow = 4 * x + (lane >> 4);         // 4 k rows of 16 chunks per instruction
      const int cb = (lane & 15) ^ (2 * (lane >> 4));
      const int q = min(q0 + 8 * cb, p.ncols - 8);  // 8 columns, inside one head (v % 8 == 0)
      const int h = q / p.v;
      b_src[i] = ((long long)h * p.r + krow) * p.v + (q - h * p.v);
    }
  }
  auto issue = [&](int k0, uint8_t* dst) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds(p.a + a_src[i] + k0, (lds_ptr)(dst + 1024 * (w + 4 * i)), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds(p.w + b_src[i] + (NN ? (long long)k0 * p.v : (long long)k0),
                                       (lds_ptr)(dst + ABYTES + 1024 * (w + 4 * i)), 16, 0, 0);
  };

  const int wm = w >> 1, wn = w & 1;
  // A / NT-B fragment: row l32 of a 32-row block, logical chunk 2 kc + half
  const int a_off = (64 * wm + l32) * 128;
  const int b_off = (64 * wn + l32) * 128;
  const int sw = lane & 7;                         // row % 8 of every fragment row
  // NN-B fragment (B^T [32 columns x 16 k] from the [k][column] tile): two
  // transposing 8-byte reads of 4 k rows each per 16-lane group
  const int G = lane >> 4, s16 = lane & 15;
  int tr_off[2];
#pragma unroll
  for (int bn = 0; bn < 2; ++bn) {
    const int krow = 8 * (G >> 1) + (s16 >> 2);
    const int chunk = 8 * wn + 4 * bn + 2 * (G & 1) + ((s16 & 3) >> 1);
    tr_off[bn] = krow * 256 + 16 * (chunk ^ (2 * (s16 >> 2))) + 8 * (s16 & 1);
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int bn = 0; bn < 2; ++bn)
#pragma unroll
    for (int bm = 0; bm < 2; ++bm)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[bn][bm][i] = 0.f;

  const int nk = p.r / BK;
  issue(0, sm);
  for (int ks = 0; ks < nk; ++ks) {
    const uint8_t* cur = sm + (ks & 1) * STAGE;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();   // stage ks landed; every wave is done with the other stage
    if (ks + 1 < nk) issue(BK * (ks + 1), sm + ((ks + 1) & 1) * STAGE);
#pragma unroll
    for (int kc = 0; kc < BK / 16; ++kc) {
      const int ch = 16 * ((2 * kc + half) ^ sw);
      u32x4 af[2], bf[2];
#pragma unroll
      for (int bm = 0; bm < 2; ++bm) af[bm] = *reinterpret_cast<const u32x4*>(cur + a_off + bm * 32 * 128 + ch);
#pragma unroll
      for (int bn = 0; bn < 2; ++bn) {
        if (!NN) {
          bf[bn] = *reinterpret_cast<const u32x4*>(cur + ABYTES + b_off + bn * 32 * 128 + ch);
        } else {
#pragma unroll
          for (int ld = 0; ld < 2; ++ld) {
            const uint8_t* src = cur + ABYTES + tr_off[bn] + (16 * kc + 4 * ld) * 256;
            const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(src));
            const u32x2 rr = __builtin_bit_cast(u32x2, r);
            bf[bn][2 * ld] = rr[0];
            bf[bn][2 * ld + 1] = rr[1];
          }
        }
      }
#pragma unroll
      for (int bn = 0; bn < 2; ++bn)
#pragma unroll
        for (int bm = 0; bm < 2; ++bm) acc[bn][bm] = mfma32(bf[bn], af[bm], acc[bn][bm]);   // C^T += B^T A^T
    }
  }

  // epilogue: C^T block (bn, bm), lane: position 32 bm + l32, columns
  // 32 bn + 8 (i / 4) + 4 half + (i % 4) -> bf16 staging [128 positions][128 columns]
  __syncthreads();   // every wave is done with the stage buffers
#pragma unroll
  for (int bn = 0; bn < 2; ++bn)
#pragma unroll
    for (int bm = 0; bm < 2; ++bm)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int m = 64 * wm + 32 * bm + l32;
        const int nn = 64 * wn + 32 * bn + 8 * qd + 4 * half;
        u32x2 v;
        v[0] = pack_bf16(acc[bn][bm][4 * qd], acc[bn][bm][4 * qd + 1]);
        v[1] = pack_bf16(acc[bn][bm][4 * qd + 2], acc[bn][bm][4 * qd + 3]);
        *reinterpret_cast<u32x2*>(sm + m * CP + nn * 2) = v;
      }
  __syncthreads();
#pragma unroll
  for (int rd = 0; rd < BM * BN / 8 / 256; ++rd) {
    const int e = tid + 256 * rd;
    const int row = e >> 4, ch = e & 15;
    const u32x4 val = *reinterpret_cast<const u32x4*>(sm + row * CP + 16 * ch);
    const long long t = t0 + row;
    const int q = q0 + 8 * ch;
    if (t < p.T && q < p.ncols) {
      if (NN) {
        st16(p.out + t * p.ncols + q, val);
      } else {
        const int h = q / p.n, j = q - h * p.n;     // n % 8 == 0: the 8 columns share a head
        st16(p.out + (t * p.H + h) * (p.n + p.rope) + j, val);
      }
    }
  }
}

// K[t, h, n:n+rope] = k_pe[t, :], 16 bytes per thread.
__global__ __launch_bounds__(256) void rope_copy_bf16_kernel(const uint16_t* __restrict__ k_pe, uint16_t* __restrict__ Kout,
                                                             long long T, int H, int n, int rope) {
  const int RC = rope / 8;
  const long long total = T * H * RC;
  for (long long o = blockIdx.x * 256LL + threadIdx.x; o < total; o += (long long)gridDim.x * 256) {
    const int ch = (int)(o % RC);
    const long long th = o / RC;
    const long long t = th / H;
    st16(Kout + th * (n + rope) + n + 8 * ch, ld16(k_pe + t * rope + 8 * ch));
  }
}

__global__ __launch_bounds__(256) void expand_f32_kernel(const float* __restrict__ c_kv, const float* __restrict__ k_pe,
                                                         const float* __restrict__ w_uk, const float* __restrict__ w_uv,
                                                         float* __restrict__ Kout, float* __restrict__ Vout,
                                                         long long T, int H, int r, int n, int v, int rope) {
  const int W = n + rope + v;
  const long long total = T * H * W;
  for (long long o = blockIdx.x * 256LL + threadIdx.x; o < total; o += (long long)gridDim.x * 256) {
    const int x = (int)(o % W);
    const long long th = o / W;
    const int h = (int)(th % H);
    const long long t = th / H;
    const float* ck = c_kv + t * r;
    if (x < n) {
      const float* wk = w_uk + ((long long)h * n + x) * r;
      float a = 0.f;
      for (int c = 0; c < r; ++c) a = fmaf(wk[c], ck[c], a);
      Kout[th * (n + rope) + x] = a;
    } else if (x < n + rope) {
      Kout[th * (n + rope) + x] = k_pe[t * rope + (x - n)];
    } else {
      const int e = x - n - rope;
      const float* wv = w_uv + (long long)h * r * v + e;
      float a = 0.f;
      for (int c = 0; c < r; ++c) a = fmaf(ck[c], wv[(long long)c * v], a);
      Vout[th * v + e] = a;
    }
  }
}

hipError_t materialize_kv(mla_dtype_t dt, long long T, int H, int r, int n, int v, int rope, const void* c_kv,
                          const void* k_pe, const void* w_uk, const void* w_uv, void* k, void* vout,
                          hipStream_t st) {
  if (dt == kBF16) {
    if (r % 64 != 0 || n % 64 != 0 || v % 64 != 0 || rope % 8 != 0) return hipErrorInvalidValue;
    ExpandArgs a{};
    a.a = (const uint16_t*)c_kv;
    a.T = T;
    a.H = H; a.r = r; a.n = n; a.v = v; a.rope = rope;
    a.MT = (int)((T + 127) / 128);
    for (int part = 0; part < 2; ++part) {
      a.w = (const uint16_t*)(part == 0 ? w_uk : w_uv);
      a.out = (uint16_t*)(part == 0 ? k : vout);
      a.ncols = H * (part == 0 ? n : v);
      const int nt = (a.ncols + 127) / 128;
      a.NTX = (nt + kXcds - 1) / kXcds;
      const long long n_items = (long long)kXcds * a.MT * a.NTX;
      if (n_items > (1LL << 30)) return hipErrorInvalidValue;
      a.n_items = (int)n_items;
      if (part == 0)
        hipLaunchKernelGGL(expand_gemm_kernel<false>, dim3((unsigned)n_items), dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL(expand_gemm_kernel<true>, dim3((unsigned)n_items), dim3(256), 0, st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || rope == 0) return e;
    const long long tot = T * H * (rope / 8);
    const long long blocks = (tot + 255) / 256;
    hipLaunchKernelGGL(rope_copy_bf16_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, st,
                       (const uint16_t*)k_pe, (uint16_t*)k, T, H, n, rope);
  } else {
    const long long total = T * H * (n + rope + v);
    const long long blocks = (total + 255) / 256;
    hipLaunchKernelGGL(expand_f32_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, st,
                       (const float*)c_kv, (const float*)k_pe, (const float*)w_uk, (const float*)w_uv, (float*)k,
                       (float*)vout, T, H, r, n, v, rope);
  }
  return hipGetLastError();
}

}  // namespace mla
