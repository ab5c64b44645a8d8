// mla_device.h -- device-side building blocks for the gfx950 (CDNA4) kernels
// of libmla: vector types, MFMA wrappers, bfloat16 conversion and packing, an
// LDS-only workgroup barrier, XCD-aware work mapping and the split-KV plan
// decode shared by the attention and merge kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;   // CDNA wavefront width
constexpr int kXcds = 8;    // MI355X: 8 accelerator complex dies, 32 CUs each

// ---- MFMA (bf16 inputs, fp32 accumulate) --------------------------------
// 32x32x16: A lane l holds row l%32, k = 8*(l/32)+j; B lane l holds col l%32,
// same k; C lane l holds col l%32, rows 8*(i/4) + 4*(l/32) + i%4, i < 16.
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// 16x16x32: A lane l holds row l%16, k = 8*(l/16)+j; B lane l holds col l%16,
// same k; C lane l holds col l%16, rows 4*(l/16) + i, i < 4.
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 16x16x128 fp8 (E4M3) with block scales, gfx950: A lane l holds row l%16, and
// its 32 bytes are k = 16*(l/16) + j (bytes j < 16) and k = 64 + 16*(l/16) + j - 16
// (bytes j >= 16); B lane l holds col l%16, same k; C as mfma16.  The E8M0
// scale of A lane l (2^(s - 127)) multiplies row l%16 over k block l/16 (k in
// 32*(l/16) .. +31), and likewise for B and its column.
typedef int i32x8 __attribute__((ext_vector_type(8)));
// SEL_B picks the byte of scale_b that holds B's scale (so four scales can share
// a register).
template <int SEL_B = 0>
__device__ __forceinline__ f32x4 mfma16_f8(i32x8 a, i32x8 b, f32x4 c, int scale_a, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, scale_a, SEL_B, scale_b);
}

// ---- E4M3 ------------------------------------------------------------------
// Smallest k with a <= 448 x 2^k for a float a >= 0 (exact, from the bits):
// a = f x 2^E with f in [1, 2); 448 = 1.75 x 2^8.
__device__ __forceinline__ int e4m3_scale_exponent(float a) {
  if (!(a > 0.f)) return 0;
  const uint32_t b = __float_as_uint(a);
  const int e = (int)((b >> 23) & 0xffu);
  if (e == 0) return -126;                            // float32 subnormal: the floor of the range
  const int E = e - 127;
  const int k = E - 8 + ((b & 0x7fffffu) > 0x600000u ? 1 : 0);
  return k < -126 ? -126 : (k > 127 ? 127 : k);
}

// max |x| over the 32 bf16 values of v[0..3], as the bf16 bit pattern of the
// magnitude: with the sign bits cleared, the patterns of non-NaN values order
// as unsigned integers, so two 16-bit maxima per instruction.  A NaN orders
// above infinity (the block's scale is then irrelevant: the row's scores are
// NaN either way).
__device__ __forceinline__ uint32_t absmax32(const u32x4 (&v)[4]) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 m = {0, 0};
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, v[c][i] & 0x7fff7fffu));
  return m[0] > m[1] ? m[0] : m[1];
}
// e4m3_scale_exponent of the float whose bf16 pattern is the magnitude m (as
// absmax32 gives it), without branches: the smallest k with m <= 448 x 2^k,
// clamped to [-126, 127]; 0 for a zero block and for NaN.  448 = 1.75 x 2^8, so
// k = E - 8, one more when the 7 mantissa bits exceed those of 1.75 (0x60).
__device__ __forceinline__ int e4m3_scale_exponent_bf16(uint32_t m) {
  const int k = max((int)(m >> 7) - 127 - 8 + ((m & 0x7fu) > 0x60u ? 1 : 0), -126);
  return (m == 0u || m > 0x7f80u) ? 0 : k;
}
// 8 bf16 values -> 8 E4M3 codes of x / s (nearest, ties to even; the division
// by a power of two is exact, so this is the rounding of x / s itself).  Each
// conversion fills the low half of a word; byte permutes pair those halves.
__device__ __forceinline__ uint32_t e4m3x2(uint32_t v, float s) {
  typedef short s16x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(
                                          __builtin_bit_cast(s16x2, v), __builtin_bit_cast(bf16x2, v), s, false));
}
__device__ __forceinline__ u32x2 e4m3x8(u32x4 v, float s) {
  return u32x2{__builtin_amdgcn_perm(e4m3x2(v[1], s), e4m3x2(v[0], s), 0x05040100u),
               __builtin_amdgcn_perm(e4m3x2(v[3], s), e4m3x2(v[2], s), 0x05040100u)};
}

// ---- bfloat16 ----------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// acc + lo + hi of a packed bf16 pair, in one dot-product instruction (weights 1, 1)
__device__ __forceinline__ float add_bf16x2(uint32_t w, float acc) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), one, acc, false);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// Round-to-nearest-even pack of two floats: one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2 v = __builtin_convertvector((float __attribute__((ext_vector_type(2)))){lo, hi}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}
// A pointer that is the same in every lane, moved to scalar registers so that
// address arithmetic on it stays on the scalar unit.
__device__ __forceinline__ const uint16_t* uniform_ptr(const uint16_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint16_t*>(((uint64_t)hi << 32) | lo);
}

// ---- workgroup barrier for LDS traffic only ---------------------------------
// Orders this wave's LDS accesses around s_barrier without waiting for its
// global loads (__syncthreads() also waits for those, so a tile copy issued
// earlier would have to land first).  Data written to LDS by direct
// global -> LDS loads is not covered: wait vmcnt(0) before a full barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---- memory --------------------------------------------------------------
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// ---- work mapping ----------------------------------------------------------
// Workgroups are dispatched round-robin over the XCDs (block id b runs on XCD
// b % 8).  Give each XCD a contiguous range of work items so that items that
// share data (the row tiles of one KV split) share that XCD's L2.
__device__ __forceinline__ int xcd_item(int bid, int n_items) {
  int per = (n_items + kXcds - 1) / kXcds;
  return (bid % kXcds) * per + bid / kXcds;
}

// Split-KV plan: sequence b (Kv_b = off[b+1]-off[b] positions) is cut into
// S_b = ceil(Kv_b / chunk) splits; splits are numbered globally in sequence
// order.  decode_split maps a global split g to (b, s); every lane of the
// wave computes the same answer.  Kv_b >= 1 for every b.
struct SplitPos { int b, s, g0; };
__device__ __forceinline__ SplitPos decode_split(int g, const int32_t* __restrict__ off, int B, int chunk) {
  const int lane = threadIdx.x % kWave;
  int base = 0;
  for (int b0 = 0; b0 < B; b0 += kWave) {
    int b = b0 + lane;
    int sb = 0;
    if (b < B) sb = (off[b + 1] - off[b] + chunk - 1) / chunk;
    // inclusive prefix sum over the wave
    int incl = sb;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      int t = __shfl_up(incl, d, kWave);
      if (lane >= d) incl += t;
    }
    int excl = incl - sb;
    bool mine = (b < B) && (g >= base + excl) && (g < base + incl);
    unsigned long long m = __ballot(mine);
    if (m) {
      int src = __ffsll((long long)m) - 1;
      int ex = __shfl(excl, src, kWave);
      SplitPos p;
      p.b = b0 + src;
      p.g0 = base + ex;
      p.s = g - p.g0;
      return p;
    }
    base += __shfl(incl, kWave - 1, kWave);
  }
  SplitPos p{B, 0, base};  // unreachable for a valid g
  return p;
}

// First global split index of sequence b and its split count.
__device__ __forceinline__ void seq_splits(int b, const int32_t* __restrict__ off, int chunk, int* g0, int* sb) {
  const int lane = threadIdx.x % kWave;
  int acc = 0;
  for (int b0 = 0; b0 < b; b0 += kWave) {
    int bb = b0 + lane;
    int s = 0;
    if (bb < b) s = (off[bb + 1] - off[bb] + chunk - 1) / chunk;
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1) s += __shfl_xor(s, d, kWave);
    acc += s;
  }
  *g0 = acc;
  *sb = (off[b + 1] - off[b] + chunk - 1) / chunk;
}

}  // namespace mla
