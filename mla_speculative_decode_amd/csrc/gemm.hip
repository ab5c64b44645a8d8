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
// [H, r, v] (the expand contracts over r) store it strided: the fold's
// small-M GEMM reads those fragments transposed from LDS (ds_read_b64_tr_b16),
// the expand transposes its W_UV tiles in registers (8x8 bf16 blocks) on the
// way into LDS.  The fold is a small-M product (M = B*L rows per head): each
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
template <int MT, int KMAX>
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

hipError_t gemm_smallm(const GemmArgs& a0, hipStream_t st) {
  GemmArgs a = a0;
  if (a.K % 32 != 0 || a.K > 512 || a.N % 64 != 0) return hipErrorInvalidValue;
  const int MT = a.M <= 16 ? 16 : 64;       // rows per workgroup
  a.n_items = a.H * (a.N / 64) * ((a.M + MT - 1) / MT);
  const unsigned grid = (unsigned)(((a.n_items + kXcds - 1) / kXcds) * kXcds);
  // LDS and staging registers are sized by KMAX: small K keeps several workgroups per CU
  const int KM = a.K <= 128 ? 128 : (a.K <= 256 ? 256 : 512);
#define MLA_GEMM(M_, KM_)                                                                \
  if (MT == M_ && KM == KM_) {                                                           \
    hipLaunchKernelGGL((gemm_smallm_kernel<M_, KM_>), dim3(grid), dim3(256), 0, st, a);  \
    return hipGetLastError();                                                            \
  }
  MLA_GEMM(16, 128) MLA_GEMM(64, 128) MLA_GEMM(16, 256) MLA_GEMM(64, 256) MLA_GEMM(16, 512) MLA_GEMM(64, 512)
#undef MLA_GEMM
  return hipErrorInvalidValue;
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
// expand, bf16: C[T x H(n+v)] = c_kv[T x r] . [W_UK[h]^T | W_UV[h]]_h.
// Workgroup tile 128 positions x 128 columns, as two 64-column halves that
// each lie inside one head's K part or V part; k steps of 32.  Wave (wm, wn)
// computes rows 64wm.., half wn as 2x2 blocks of 32x32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int ab_phys(int row, int ch) { return ch ^ ((row >> 1) & 3); }

__global__ __launch_bounds__(256) void expand_bf16_kernel(const uint16_t* __restrict__ c_kv,
                                                          const uint16_t* __restrict__ w_uk,
                                                          const uint16_t* __restrict__ w_uv,
                                                          uint16_t* __restrict__ Kout, uint16_t* __restrict__ Vout,
                                                          long long T, int H, int r, int n, int v, int rope,
                                                          int CT, int n_items) {
  __shared__ __attribute__((aligned(16))) uint8_t as_[128 * 64];
  __shared__ __attribute__((aligned(16))) uint8_t bs_[128 * 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int item = xcd_item(blockIdx.x, n_items);
  if (item >= n_items) return;
  const int ct = item % CT;
  const long long t0 = (long long)(item / CT) * 128;
  const int NC = n + v;
  const int ncols = H * NC;

  int hh[2], j0[2];
  bool isK[2], act[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int col0 = ct * 128 + 64 * hf;
    act[hf] = col0 < ncols;
    const int cc = act[hf] ? col0 : 0;
    hh[hf] = cc / NC;
    const int x = cc % NC;
    isK[hf] = x < n;
    j0[hf] = isK[hf] ? x : x - n;
  }

  u32x4 ast[2];
  u32x4 bst[2][8];
  auto load = [&](int k0) {
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int C = tid + 256 * y;
      const int row = C >> 2, ch = C & 3;
      long long t = t0 + row;
      if (t >= T) t = T - 1;
      ast[y] = ld16(c_kv + t * r + k0 + 8 * ch);
    }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      if (!act[hf]) continue;
      if (isK[hf]) {
        const int col = tid >> 2, ch = tid & 3;
        bst[hf][0] = ld16(w_uk + ((long long)hh[hf] * n + j0[hf] + col) * r + k0 + 8 * ch);
      } else if (tid < 32) {
        const int kg = tid & 3, cc = tid >> 2;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          bst[hf][jj] = ld16(w_uv + ((long long)hh[hf] * r + k0 + 8 * kg + jj) * v + j0[hf] + 8 * cc);
      }
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int C = tid + 256 * y;
      const int row = C >> 2, ch = C & 3;
      st16(as_ + row * 64 + ab_phys(row, ch) * 16, ast[y]);
    }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      if (!act[hf]) continue;
      if (isK[hf]) {
        const int row = 64 * hf + (tid >> 2), ch = tid & 3;
        st16(bs_ + row * 64 + ab_phys(row, ch) * 16, bst[hf][0]);
      } else if (tid < 32) {
        const int kg = tid & 3, cc = tid >> 2;
        u32x4 tr[8];
        transpose8x8_bf16(bst[hf], tr);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int row = 64 * hf + 8 * cc + e;
          st16(bs_ + row * 64 + ab_phys(row, kg) * 16, tr[e]);
        }
      }
    }
  };

  const int wm = w >> 1, wn = w & 1;
  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][c][i] = 0.f;

  const int nks = r / 32;
  load(0);
  for (int ks = 0; ks < nks; ++ks) {
    store();
    __syncthreads();
    if (ks + 1 < nks) load(32 * (ks + 1));
    if (act[wn]) {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        u32x4 a[2], bv[2];
#pragma unroll
        for (int bm = 0; bm < 2; ++bm) {
          const int row = 64 * wm + 32 * bm + l32;
          a[bm] = *reinterpret_cast<const u32x4*>(as_ + row * 64 + ab_phys(row, 2 * kc + half) * 16);
        }
#pragma unroll
        for (int bn = 0; bn < 2; ++bn) {
          const int row = 64 * wn + 32 * bn + l32;
          bv[bn] = *reinterpret_cast<const u32x4*>(bs_ + row * 64 + ab_phys(row, 2 * kc + half) * 16);
        }
#pragma unroll
        for (int bm = 0; bm < 2; ++bm)
#pragma unroll
          for (int bn = 0; bn < 2; ++bn) acc[bm][bn] = mfma32(a[bm], bv[bn], acc[bm][bn]);
      }
    }
    __syncthreads();
  }
  if (!act[wn]) return;
  const int h = hh[wn];
#pragma unroll
  for (int bm = 0; bm < 2; ++bm)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const long long t = t0 + 64 * wm + 32 * bm + 8 * (i >> 2) + 4 * half + (i & 3);
      if (t >= T) continue;
#pragma unroll
      for (int bn = 0; bn < 2; ++bn) {
        const int j = j0[wn] + 32 * bn + l32;
        const uint16_t o = __builtin_bit_cast(uint16_t, (__bf16)acc[bm][bn][i]);
        if (isK[wn]) Kout[(t * H + h) * (n + rope) + j] = o;
        else Vout[(t * H + h) * v + j] = o;
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
    const int CT = (H * (n + v) + 127) / 128;
    const long long TT = (T + 127) / 128;
    const long long n_items = TT * CT;
    if (n_items > (1LL << 30)) return hipErrorInvalidValue;
    const unsigned grid = (unsigned)(((n_items + kXcds - 1) / kXcds) * kXcds);
    hipLaunchKernelGGL(expand_bf16_kernel, dim3(grid), dim3(256), 0, st, (const uint16_t*)c_kv,
                       (const uint16_t*)w_uk, (const uint16_t*)w_uv, (uint16_t*)k, (uint16_t*)vout, T, H, r, n, v,
                       rope, CT, (int)n_items);
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
