// attn.hip -- split-KV attention kernels of libmla and their combine passes.
//
// One kernel template serves both MLA routes (pages: "One guard, 110x off the
// verify step", section "The defect"):
//   absorbed     : every (row, head) pair of a sequence is a query of width
//                  r + rope = [q_lat | q_pe] against the shared keys
//                  [c_kv | k_pe]; the values are c_kv itself, so one latent
//                  tile, read once into LDS, serves the scores and the
//                  weighted sum of all L*H pairs (multi-query attention with a
//                  single shared key/value head);
//   materialised : each head attends over its own expanded K [T, H, n+rope]
//                  and V [T, H, v].
// Positions of a sequence are cut into splits; each workgroup takes 64 query
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
//   softmax base-2 online softmax; the two key halves of a row exchange their
//           partial maxima through LDS;
//   PV      O[64 rows x DV]: wave w owns columns w*DV/4..; P (bf16) comes from
//           LDS, V^T from an LDS copy transposed in registers on the way in.
// LDS holds one key tile row-major (kt), one value tile transposed (vt), P,
// and small exchange arrays; the next tile is prefetched into registers and
// written to kt while PV runs, and to vt right after it.

#include "mla_device.h"
#include "internal.h"

namespace mla {

// ---------------------------------------------------------------------------
// bf16 MFMA split-KV attention
// ---------------------------------------------------------------------------
struct AttnArgs {
  const uint16_t* qa;   // query part a: [B, L, H, DA]
  const uint16_t* qb;   // query part b: [B, L, H, DR]
  const uint16_t* ka;   // key-only source (see KW), row for position p at ka + p*ka_ks + head*ka_hs
  const uint16_t* vv;   // value source, row for position p at vv + p*vv_ks + head*vv_hs
  long long ka_ks, ka_hs, vv_ks, vv_hs;
  const int32_t* off;   // [B+1] device offsets
  float* ws_o;          // [G][rows_total][DV]
  float* ws_ml;         // [G][rows_total][2]
  int B, L, H;
  int hpr;              // heads per row slot (absorbed: H, materialised: 1)
  int rows_slot;        // query rows per (sequence, head slot)
  int head_slots;       // absorbed: 1, materialised: H
  int row_tiles;        // ceil(rows_slot / 64)
  int chunk;            // positions per split (multiple of 64)
  int n_items;
  int rows_total;       // L*H
  float sl2;            // scale * log2(e)
};

__device__ __forceinline__ int kt_phys(int key, int ch) { return ch ^ ((key & 7) ^ ((key >> 3) & 7)); }
__device__ __forceinline__ int row_phys(int row, int ch) { return ch ^ (row & 7); }

// DA: width of query part a (= width of the V source when VK); DR: query part
// b width; DV: value width; VK: values are the first DA key columns (absorbed).
template <int DA, int DR, int DV, bool VK>
__global__ __launch_bounds__(256, 1) void attn_bf16_kernel(AttnArgs p) {
  constexpr int D = DA + DR;
  constexpr int BM = 64, BN = 64, NT = 256;
  constexpr int DCH = D / 16;             // 16-wide k steps of the score MFMA
  constexpr int KTC = D / 8;              // 16-byte chunks per kt row
  constexpr int KW = VK ? DR : D;         // width of the key-only source
  constexpr int KOFF = VK ? DA / 8 : 0;   // first kt chunk the key-only source fills
  constexpr int NKC = BN * (KW / 8);      // key-only chunks per tile
  constexpr int NKC_T = (NKC + NT - 1) / NT;
  constexpr int NVU = DV;                 // value units: (DV/8 column chunks) x (BN/8 key groups)
  constexpr int NVU_T = (NVU + NT - 1) / NT;
  constexpr int CPW = DV / 4;             // value columns per wave
  constexpr int NCB = CPW / 32;           // 32-column MFMA blocks per wave
  static_assert(D % 64 == 0 && DV % 128 == 0 && (!VK || DA == DV), "unsupported geometry");

  __shared__ __attribute__((aligned(16))) uint8_t kt[BN * D * 2];
  __shared__ __attribute__((aligned(16))) uint8_t vt[DV * BN * 2];
  __shared__ __attribute__((aligned(16))) uint8_t pl[BM * BN * 2];
  __shared__ float red[2 * BM];
  __shared__ __attribute__((aligned(16))) float al[BM];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int item = xcd_item(blockIdx.x, p.n_items);
  if (item >= p.n_items) return;
  const int rt = item % p.row_tiles;
  const int tmp = item / p.row_tiles;
  const int hs = tmp % p.head_slots;
  const int g = tmp / p.head_slots;
  const SplitPos sp = decode_split(g, p.off, p.B, p.chunk);
  const int b = sp.b;
  const long long p0 = p.off[b];
  const int Kv = p.off[b + 1] - p.off[b];
  const int k0 = sp.s * p.chunk;
  const int k1 = min(Kv, k0 + p.chunk);
  const int idx0 = rt * BM;
  const int nrows = min(BM, p.rows_slot - idx0);

  const uint16_t* kab = p.ka + (long long)hs * p.ka_hs;
  const uint16_t* vvb = p.vv + (long long)hs * p.vv_hs;

  // ---- score-phase identity: wave (wk, wr), query row rq of the tile -------
  const int wk = w & 1, wr = w >> 1;
  const int rq = 32 * wr + l32;
  const bool rq_ok = rq < nrows;
  int kend = 0;   // positions this row may see within the split (relative to sequence start)
  u32x4 qf[DCH];
  {
    const int idx = idx0 + rq;
    const int i = idx / p.hpr;
    const int h = hs + idx % p.hpr;
    const long long flat = ((long long)b * p.L + i) * p.H + h;
    kend = min(k1, Kv - p.L + i + 1);
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

  // ---- staging registers for the next tile --------------------------------
  u32x4 vst[NVU_T > 0 ? NVU_T : 1][8];
  u32x4 kst[NKC_T > 0 ? NKC_T : 1];

  auto load_tile = [&](int t0) {
#pragma unroll
    for (int x = 0; x < NVU_T; ++x) {
      const int U = tid + NT * x;
      if (U < NVU) {
        const int kg = U & 7, c = U >> 3;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int key = min(t0 + 8 * kg + j, k1 - 1);
          vst[x][j] = ld16(vvb + (p0 + key) * p.vv_ks + 8 * c);
        }
      }
    }
#pragma unroll
    for (int x = 0; x < NKC_T; ++x) {
      const int C = tid + NT * x;
      if (C < NKC) {
        constexpr int KC = KW > 0 ? KW / 8 : 1;
        const int key = C / KC, ch = C % KC;
        const int kk = min(t0 + key, k1 - 1);
        kst[x] = ld16(kab + (p0 + kk) * p.ka_ks + 8 * ch);
      }
    }
  };
  auto write_kt = [&]() {
#pragma unroll
    for (int x = 0; x < NKC_T; ++x) {
      const int C = tid + NT * x;
      if (C < NKC) {
        constexpr int KC = KW > 0 ? KW / 8 : 1;
        const int key = C / KC, ch = KOFF + C % KC;
        st16(kt + key * (D * 2) + kt_phys(key, ch) * 16, kst[x]);
      }
    }
    if (VK) {
#pragma unroll
      for (int x = 0; x < NVU_T; ++x) {
        const int U = tid + NT * x;
        if (U < NVU) {
          const int kg = U & 7, c = U >> 3;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int key = 8 * kg + j;
            st16(kt + key * (D * 2) + kt_phys(key, c) * 16, vst[x][j]);
          }
        }
      }
    }
  };
  auto write_vt = [&]() {
#pragma unroll
    for (int x = 0; x < NVU_T; ++x) {
      const int U = tid + NT * x;
      if (U < NVU) {
        const int kg = U & 7, c = U >> 3;
        u32x4 tr[8];
        transpose8x8_bf16(vst[x], tr);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int row = 8 * c + e;
          st16(vt + row * (BN * 2) + row_phys(row, kg) * 16, tr[e]);
        }
      }
    }
  };

  // ---- running state ------------------------------------------------------
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 O[2][NCB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) O[rb][cb][i] = 0.f;

  load_tile(k0);
  write_kt();
  write_vt();
  if (k0 + BN < k1) load_tile(k0 + BN);
  __syncthreads();

  for (int t0 = k0; t0 < k1; t0 += BN) {
    const bool has_next = t0 + BN < k1;
    // ---- scores: S^T block [32 keys x 32 rows] --------------------------
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    {
      const int key = 32 * wk + l32;
      const uint8_t* krow = kt + key * (D * 2);
#pragma unroll
      for (int c = 0; c < DCH; ++c) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(krow + kt_phys(key, 2 * c + half) * 16);
        acc = mfma32(a, qf[c], acc);
      }
    }
    float s[16];
    float pmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = t0 + 32 * wk + 8 * (i >> 2) + 4 * half + (i & 3);
      s[i] = key < kend ? acc[i] * p.sl2 : -INFINITY;
      pmax = fmaxf(pmax, s[i]);
    }
    pmax = fmaxf(pmax, __shfl_xor(pmax, 32, 64));
    if (half == 0) red[wk * BM + rq] = pmax;
    __syncthreads();  // (1) scores done: kt free; partial maxima visible

    {
      const float tmax = fmaxf(pmax, red[(1 - wk) * BM + rq]);
      const float m_new = fmaxf(m_run, tmax);
      const bool none = (m_new == -INFINITY);
      const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = none ? 0.f : __builtin_amdgcn_exp2f(s[i] - m_new);
        psum += s[i];
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x2 v;
        v[0] = pack_bf16(s[4 * q + 0], s[4 * q + 1]);
        v[1] = pack_bf16(s[4 * q + 2], s[4 * q + 3]);
        *reinterpret_cast<u32x2*>(pl + rq * (BN * 2) + row_phys(rq, 4 * wk + q) * 16 + 8 * half) = v;
      }
      if (wk == 0 && half == 0) al[rq] = alpha;
    }
    __syncthreads();  // (2) P and rescale factors visible

    if (has_next) write_kt();  // next keys into kt while PV runs

    // ---- PV: O[64 rows x CPW] for this wave's columns ----------------------
    {
      bool any = false;
      f32x4 alv[2][4];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          alv[rb][q] = *reinterpret_cast<const f32x4*>(&al[32 * rb + 8 * q + 4 * half]);
          any |= (alv[rb][q][0] != 1.f) | (alv[rb][q][1] != 1.f) | (alv[rb][q][2] != 1.f) |
                 (alv[rb][q][3] != 1.f);
        }
      if (__ballot(any)) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) O[rb][cb][i] *= alv[rb][i >> 2][i & 3];
      }
      const int col0 = w * CPW;
#pragma unroll
      for (int kc = 0; kc < BN / 16; ++kc) {
        u32x4 a[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const int row = 32 * rb + l32;
          a[rb] = *reinterpret_cast<const u32x4*>(pl + row * (BN * 2) + row_phys(row, 2 * kc + half) * 16);
        }
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const int col = col0 + 32 * cb + l32;
          const u32x4 bv = *reinterpret_cast<const u32x4*>(vt + col * (BN * 2) + row_phys(col, 2 * kc + half) * 16);
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) O[rb][cb] = mfma32(a[rb], bv, O[rb][cb]);
        }
      }
    }
    __syncthreads();  // (3) PV done: vt and pl free; next kt complete
    if (has_next) {
      write_vt();  // visible to PV(t+1) through barriers (1) and (2) of the next tile
      if (t0 + 2 * BN < k1) load_tile(t0 + 2 * BN);
    }
  }

  // ---- epilogue: row sums, partial results ---------------------------------
  const float lw = l_run + __shfl_xor(l_run, 32, 64);
  __syncthreads();
  if (half == 0) red[wk * BM + rq] = lw;
  __syncthreads();
  const long long gro = (long long)g * p.rows_total;
  if (wk == 0 && half == 0 && rq_ok) {
    const int prow = hs * p.rows_slot + idx0 + rq;
    p.ws_ml[(gro + prow) * 2 + 0] = m_run;
    p.ws_ml[(gro + prow) * 2 + 1] = red[rq] + red[BM + rq];
  }
  const int col0 = w * CPW;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 32 * rb + 8 * (i >> 2) + 4 * half + (i & 3);
      if (row < nrows) {
        const int prow = hs * p.rows_slot + idx0 + row;
        float* dst = p.ws_o + (gro + prow) * DV + col0 + l32;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) dst[32 * cb] = O[rb][cb][i];
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

// out[b,i,h,:] = sum_s w_s o_s  (materialised route; any dtype, float32 partials).
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
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
      a = fmaf(__builtin_amdgcn_exp2f(m - M), ws_o[((long long)(g0 + s) * rows_total + prow) * DV + c], a);
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

// Absorbed route, bf16: merge the splits while building the MFMA A operand
// (each lane reads exactly the latent slice it feeds), then multiply by the
// W_UV tile (transposed into LDS in registers).  Workgroup = (sequence, 16
// query rows, head, 64 output columns); wave w covers latent rows
// w*R/4 .. (w+1)*R/4 and the four waves' partial products are summed in LDS.
template <int R>
__global__ __launch_bounds__(256) void combine_upproj_bf16_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
                                                                  const int32_t* __restrict__ off, int B, int L, int H, int V,
                                                                  int chunk, const uint16_t* __restrict__ w_uv,
                                                                  float* __restrict__ out, int n_items) {
  constexpr int KW = R / 4;          // latent rows per wave
  constexpr int KCH = KW / 8;        // 16-byte chunks per wt row
  __shared__ __attribute__((aligned(16))) uint8_t wt[4][64 * KW * 2];
  __shared__ __attribute__((aligned(16))) float red[4][16 * 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int item = xcd_item(blockIdx.x, n_items);
  if (item >= n_items) return;
  const int CT = V / 64, RT = (L + 15) / 16;
  const int ct = item % CT;
  int tmp = item / CT;
  const int h = tmp % H; tmp /= H;
  const int rt = tmp % RT;
  const int b = tmp / RT;
  const int rows_total = L * H;
  const int kw0 = w * KW;

  // W_UV[h][kw0 + k][ct*64 + col] -> wt[w][col][k] (k contiguous)
  const uint16_t* wsrc = w_uv + ((long long)h * R + kw0) * V + ct * 64;
  for (int U = lane; U < (KW / 8) * 8; U += 64) {
    const int kg = U >> 3, cc = U & 7;
    u32x4 in[8], tr[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) in[j] = ld16(wsrc + (long long)(8 * kg + j) * V + 8 * cc);
    transpose8x8_bf16(in, tr);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int col = 8 * cc + e;
      st16(&wt[w][col * KW * 2 + ((kg ^ (col & 7)) * 16)], tr[e]);
    }
  }

  int g0, S;
  seq_splits(b, off, chunk, &g0, &S);
  const int r16 = lane & 15, kq = lane >> 4;
  const int i = rt * 16 + r16;
  const bool ok = i < L;
  const int prow = i * H + h;
  float M = -INFINITY, inv = 0.f;
  if (ok) merge_stats(ws_ml + ((long long)g0 * rows_total + prow) * 2, rows_total, S, &M, &inv);
  __syncthreads();

  f32x4 acc[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kc = 0; kc < KW / 32; ++kc) {
    const int k = kw0 + 32 * kc + 8 * kq;
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (ok) {
      for (int s = 0; s < S; ++s) {
        const float m = ws_ml[((long long)(g0 + s) * rows_total + prow) * 2];
        if (m == -INFINITY) continue;
        const float wgt = __builtin_amdgcn_exp2f(m - M) * inv;
        const float* src = ws_o + ((long long)(g0 + s) * rows_total + prow) * R + k;
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(src);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 4);
        o[0] = fmaf(wgt, x0[0], o[0]); o[1] = fmaf(wgt, x0[1], o[1]);
        o[2] = fmaf(wgt, x0[2], o[2]); o[3] = fmaf(wgt, x0[3], o[3]);
        o[4] = fmaf(wgt, x1[0], o[4]); o[5] = fmaf(wgt, x1[1], o[5]);
        o[6] = fmaf(wgt, x1[2], o[6]); o[7] = fmaf(wgt, x1[3], o[7]);
      }
    }
    u32x4 a;
    a[0] = pack_bf16(o[0], o[1]); a[1] = pack_bf16(o[2], o[3]);
    a[2] = pack_bf16(o[4], o[5]); a[3] = pack_bf16(o[6], o[7]);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int col = 16 * cb + r16;
      const int ch = 4 * kc + kq;
      const u32x4 bv = *reinterpret_cast<const u32x4*>(&wt[w][col * KW * 2 + ((ch ^ (col & 7)) * 16)]);
      acc[cb] = mfma16(a, bv, acc[cb]);
    }
  }
  // C layout: lane holds col 16cb + lane%16, rows 4*(lane/16) + x
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int x = 0; x < 4; ++x) red[w][(4 * kq + x) * 64 + 16 * cb + r16] = acc[cb][x];
  __syncthreads();
  for (int e = tid; e < 16 * 64; e += 256) {
    const int rr = e >> 6, col = e & 63;
    const int ii = rt * 16 + rr;
    if (ii < L) {
      const float v = red[0][e] + red[1][e] + red[2][e] + red[3][e];
      out[(((long long)b * L + ii) * H + h) * V + ct * 64 + col] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static inline unsigned grid_xcd(int n_items) { return (unsigned)(((n_items + kXcds - 1) / kXcds) * kXcds); }

template <int DA, int DR, int DV, bool VK>
static hipError_t launch_attn(const AttnArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((attn_bf16_kernel<DA, DR, DV, VK>), dim3(grid_xcd(a.n_items)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t absorbed_attn_bf16(const AbsorbedLaunch& q, hipStream_t st) {
  AttnArgs a{};
  a.qa = (const uint16_t*)q.q_lat; a.qb = (const uint16_t*)q.q_pe;
  a.ka = (const uint16_t*)q.k_pe; a.ka_ks = q.rope; a.ka_hs = 0;
  a.vv = (const uint16_t*)q.c_kv; a.vv_ks = q.r; a.vv_hs = 0;
  a.off = q.off_dev; a.ws_o = q.ws_o; a.ws_ml = q.ws_ml;
  a.B = q.B; a.L = q.L; a.H = q.H; a.hpr = q.H; a.rows_slot = q.L * q.H; a.head_slots = 1;
  a.row_tiles = q.plan.row_tiles; a.chunk = q.plan.chunk; a.n_items = q.plan.n_items;
  a.rows_total = q.L * q.H; a.sl2 = q.scale * 1.4426950408889634f;
  if (q.r != 512) return hipErrorInvalidValue;
  switch (q.rope) {
    case 0:  return launch_attn<512, 0, 512, true>(a, st);
    case 64: return launch_attn<512, 64, 512, true>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t materialized_attn_bf16(const MaterializedLaunch& q, hipStream_t st) {
  AttnArgs a{};
  const int D = q.n + q.rope;
  a.qa = (const uint16_t*)q.q_nope; a.qb = (const uint16_t*)q.q_pe;
  a.ka = (const uint16_t*)q.k; a.ka_ks = (long long)q.H * D; a.ka_hs = D;
  a.vv = (const uint16_t*)q.v; a.vv_ks = (long long)q.H * q.v_dim; a.vv_hs = q.v_dim;
  a.off = q.off_dev; a.ws_o = q.ws_o; a.ws_ml = q.ws_ml;
  a.B = q.B; a.L = q.L; a.H = q.H; a.hpr = 1; a.rows_slot = q.L; a.head_slots = q.H;
  a.row_tiles = q.plan.row_tiles; a.chunk = q.plan.chunk; a.n_items = q.plan.n_items;
  a.rows_total = q.L * q.H; a.sl2 = q.scale * 1.4426950408889634f;
  // The kernel sees the query as [q_nope | q_pe] of width n + rope and K rows
  // of the same width; DA = n, DR = rope.
#define MLA_MAT(N, RP, VD) \
  if (q.n == N && q.rope == RP && q.v_dim == VD) return launch_attn<N, RP, VD, false>(a, st);
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
    a.off = q.off_dev; a.ws_o = q.ws_o; a.ws_ml = q.ws_ml;
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
    a.off = q.off_dev; a.ws_o = q.ws_o; a.ws_ml = q.ws_ml;
    a.B = q.B; a.L = q.L; a.H = q.H; a.hpr = 1; a.rows_slot = q.L; a.head_slots = q.H;
    a.chunk = q.plan.chunk; a.rows_total = q.L * q.H; a.sl2 = q.scale * 1.4426950408889634f;
    a.n_items = q.plan.n_splits * a.head_slots * a.rows_slot;
  }
  if (a.DA + a.DR > kF32MaxD || a.DV > kF32MaxDV) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_f32_kernel, dim3(a.n_items), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t combine_materialized(const MaterializedLaunch& q, float* out, hipStream_t st) {
  hipLaunchKernelGGL(combine_kernel, dim3(q.B * q.L * q.H), dim3(256), 0, st, (const float*)q.ws_o,
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
  const int n_items = q.B * ((q.L + 15) / 16) * q.H * (q.v_dim / 64);
  hipLaunchKernelGGL(combine_upproj_bf16_kernel<512>, dim3(grid_xcd(n_items)), dim3(256), 0, st,
                     (const float*)q.ws_o, (const float*)q.ws_ml, q.off_dev, q.B, q.L, q.H, q.v_dim,
                     q.plan.chunk, (const uint16_t*)q.w_uv, out, n_items);
  return hipGetLastError();
}

}  // namespace mla
