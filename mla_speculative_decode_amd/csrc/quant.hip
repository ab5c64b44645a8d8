// quant.hip -- fp8 (OCP E4M3) form of the latent cache.
//
// The pages test a "quantised latent form" of the cache without defining it
// (mlx-lm PR #1817, section "Tests").  The form built here: each cached
// position's row [c_kv | k_pe] is stored as E4M3 codes (1 sign bit, 4 exponent
// bits with bias 7, 3 mantissa bits; subnormals m x 2^-9; no infinities;
// largest finite value 448) with one power-of-two scale 2^k per position, the
// smallest with max|x| <= 448 x 2^k (k in [-126, 127]; 0 for an all-zero row).
// x / 2^k is then exact in float32, and every dequantised value code x 2^k is
// exact in bfloat16, so attention kernels can expand the codes into bf16 tiles
// without rounding.  Encoding rounds to the nearest E4M3 value, ties to the
// even code; a negative value that rounds to zero gets code 0.

#include "mla_device.h"
#include "internal.h"

namespace mla {

// Nearest E4M3 code of y (|y| <= 448 after saturation), ties to the even code.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const float a = fminf(fabsf(y), 448.f);
  uint32_t code;
  if (a < 0.015625f) {                                // below 2^-6: subnormal grid m x 2^-9
    code = (uint32_t)rintf(a * 512.f);                 // exact scaling, round half to even; 8 -> 0x08 = 2^-6
  } else {
    const uint32_t b = __float_as_uint(a);
    int E = (int)((b >> 23) & 0xffu) - 127;            // -6 .. 8
    const uint32_t mant = b & 0x7fffffu;
    uint32_t q = mant >> 20;                           // 3 kept mantissa bits
    const uint32_t rem = mant & 0xfffffu, half = 0x80000u;
    q += (rem > half || (rem == half && (q & 1u))) ? 1u : 0u;
    if (q == 8u) { q = 0u; ++E; }
    code = ((uint32_t)(E + 7) << 3) | q;
    if (code > 0x7eu) code = 0x7eu;                   // saturate at 448 (0x7f is NaN)
  }
  if (y < 0.f && code != 0u) code |= 0x80u;
  return code;
}

// One wave per cached position: 16-byte chunks of the bf16 row (lane l takes
// chunk l, lanes 0..W-65 also chunk 64 + l), the row maximum by a wave
// reduction, then 8 codes per chunk.
__global__ __launch_bounds__(256) void quantize_latent_kernel(const uint16_t* __restrict__ c_kv,
                                                              const uint16_t* __restrict__ k_pe,
                                                              uint8_t* __restrict__ codes, float* __restrict__ scales,
                                                              long long T, int r, int rope) {
  const int lane = threadIdx.x & 63;
  const long long t = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int RC = r / 8, NC = (r + rope) / 8;           // 16-byte chunks: latent, whole row
  u32x4 v[2];
  float amax = 0.f;
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int ch = lane + 64 * x;
    v[x] = u32x4{0u, 0u, 0u, 0u};
    if (ch < NC) {
      v[x] = ch < RC ? ld16(c_kv + t * r + 8 * ch) : ld16(k_pe + t * rope + 8 * (ch - RC));
#pragma unroll
      for (int q = 0; q < 4; ++q) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(v[x][q])), fabsf(bf16_hi(v[x][q]))));
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, kWave));
  const int k = e4m3_scale_exponent(amax);
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int ch = lane + 64 * x;
    if (ch < NC) {
      uint32_t w[2] = {0u, 0u};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t c0 = e4m3_encode(ldexpf(bf16_lo(v[x][q]), -k));
        const uint32_t c1 = e4m3_encode(ldexpf(bf16_hi(v[x][q]), -k));
        w[q >> 1] |= (c0 | (c1 << 8)) << (16 * (q & 1));
      }
      *reinterpret_cast<uint2*>(codes + t * (r + rope) + 8 * ch) = make_uint2(w[0], w[1]);
    }
  }
  if (lane == 0) scales[t] = __uint_as_float((uint32_t)(k + 127) << 23);
}

hipError_t quantize_latent_fp8(long long T, int r, int rope, const void* c_kv, const void* k_pe, void* codes,
                               float* scales, hipStream_t st) {
  if (r % 8 != 0 || rope % 8 != 0 || (r + rope) / 8 > 128) return hipErrorInvalidValue;
  const long long blocks = (T + 3) / 4;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quantize_latent_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const uint16_t*)c_kv,
                     (const uint16_t*)k_pe, (uint8_t*)codes, scales, T, r, rope);
  return hipGetLastError();
}

}  // namespace mla
