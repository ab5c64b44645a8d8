// bench_peaks.hip -- the two achievable peaks the benchmark reports fractions
// against, measured on the running GPU (part of libmla_bench.so, used only by
// bench.py): a streaming read of a large buffer (HBM) and a dense stream of
// independent bf16 32x32x16 MFMAs.  Also two LDS probes behind the split
// kernels' LDS layouts: which lanes of one read instruction LDS serves in the
// same cycle, and the cycles of the score-fragment and transposed V reads under
// a given row layout.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Each workgroup streams one contiguous chunk of the buffer: per round its 256
// threads read 8 x 4 KB with 16-byte non-temporal loads (8 KB in flight per
// wave).  On MI355X this pattern reads about 7 TB/s; a grid-stride pattern
// (each load a whole grid apart) or ordinary cached loads stay near 5.5-6.3.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, long long n16,
                                                          uint32_t* __restrict__ sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const long long per = (n16 + gridDim.x - 1) / gridDim.x;
  const long long b0 = (long long)blockIdx.x * per;
  const long long b1 = b0 + per < n16 ? b0 + per : n16;
  long long i = b0 + threadIdx.x;
  for (; i + 7 * 256 < b1; i += 8 * 256) {
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __builtin_nontemporal_load(p + i + j * 256);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= v[j];
  }
  for (; i < b1; i += 256) acc ^= p[i];
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) sink[0] = acc.x;   // keeps the loads live
}

// Four independent accumulator chains per wave.
__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float* __restrict__ sink) {
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(1e-3f * (float)((threadIdx.x + j) & 7));
    b[j] = (__bf16)(1e-3f * (float)((threadIdx.x * 3 + j) & 7));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) s += c0[k] + c1[k] + c2[k] + c3[k];
  if (s == 1.2345f) sink[0] = s;   // keeps the products live
}


// ---- LDS probes: one 512-thread workgroup per CU (136 KB of LDS each), 8 waves,
// `iters` rounds of 16 reads 1 KB apart (the same banks, distinct addresses);
// cycles per wave from s_memtime.  Every address stays below 48 KB.
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr int kLdsProbeBytes = 139264;

template <int OP>
__device__ __forceinline__ uint32_t lds_read(const uint8_t* a) {
  if (OP == 0) { const u32x4 r = *reinterpret_cast<const u32x4*>(a); return r[0] ^ r[3]; }
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(a));
  const u32x2 rr = __builtin_bit_cast(u32x2, r);
  return rr[0] ^ rr[1];
}

// Lane pair (OP 0: ds_read_b128, 1: ds_read_b64_tr_b16): every
// lane reads one broadcast address except lanes li and lj, lane li at bank set
// 5 (bytes 80..95 of a 256-byte bank row), lane lj at bank set 5 (same = 1) or
// 9, each at another address.  Same-set pairs served in one cycle conflict.
template <int OP>
__global__ __launch_bounds__(512, 1) void lds_pair_kernel(int li, int lj, int same, int iters,
                                                         unsigned long long* __restrict__ cycles,
                                                         uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsProbeBytes];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < kLdsProbeBytes / 16; i += 512) reinterpret_cast<u32x4*>(lds)[i] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  int base = 0;
  if (lane == li) base = 16 * 5 + 4096;
  if (lane == lj) base = 16 * (same ? 5 : 9) + 8192;
  base += 20480 * (w & 1);
  uint32_t acc = 0;
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    int a = base;
    asm volatile("" : "+v"(a));
    uint32_t x[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) x[k] = lds_read<OP>(lds + a + 1024 * k);
#pragma unroll
    for (int k = 0; k < 16; ++k) acc ^= x[k];
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  if (lane == 0) cycles[blockIdx.x * 8 + w] = t1 - t0;
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

// The bf16 split kernel's two heavy read patterns over latent rows of `lrb`
// bytes whose 16-byte chunk index is XOR-ed with 2 ((row >> 2) & 1) when swz:
// PAT 0, score fragments (ds_read_b128: rows 16 (w & 1) + lane % 16, chunk
// 4 ks + lane / 16); PAT 1, transposed V reads (ds_read_b64_tr_b16: rows
// 16 kc + 4 ld + 8 (lane / 32) + lane % 16 / 4, bytes 256 (w & 3) + 32 (lane / 16
// & 1) + 8 (lane & 3) + 64 cb).
template <int PAT>
__global__ __launch_bounds__(512, 1) void lds_layout_kernel(int lrb, int swz, int iters,
                                                           unsigned long long* __restrict__ cycles,
                                                           uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsProbeBytes];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < kLdsProbeBytes / 16; i += 512) reinterpret_cast<u32x4*>(lds)[i] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  auto at = [&](int row, int byte) {
    int c = byte >> 4;
    if (swz) c ^= ((row >> 2) & 1) << 1;
    return row * lrb + 16 * c + (byte & 15);
  };
  int addr[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    if (PAT == 0) {
      addr[k] = at(16 * (w & 1) + (lane & 15), 64 * k + 16 * (lane >> 4));
    } else {
      const int kc = k >> 3, ld = (k >> 2) & 1, cb = k & 3, G = lane >> 4, s16 = lane & 15;
      addr[k] = at(16 * kc + 4 * ld + 8 * (G >> 1) + (s16 >> 2), 256 * (w & 3) + 32 * (G & 1) + 8 * (s16 & 3) + 64 * cb);
    }
  }
  uint32_t acc = 0;
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k) asm volatile("" : "+v"(addr[k]));   // in place: no copies
    uint32_t x[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) x[k] = lds_read<PAT == 0 ? 0 : 1>(lds + addr[k]);
#pragma unroll
    for (int k = 0; k < 16; ++k) acc ^= x[k];
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  if (lane == 0) cycles[blockIdx.x * 8 + w] = t1 - t0;
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

double mean_cycles(const unsigned long long* dev, hipStream_t st) {
  unsigned long long h[256 * 8];
  if (hipMemcpyAsync(h, dev, sizeof(h), hipMemcpyDeviceToHost, st) != hipSuccess) return -1.0;
  if (hipStreamSynchronize(st) != hipSuccess) return -1.0;
  double s = 0.0;
  for (unsigned long long x : h) s += (double)x;
  return s / (256 * 8);
}
}  // namespace

extern "C" {

// HBM read bandwidth: `reps` reads of `bytes` (a multiple of 16) at `buf`, timed
// with HIP events on `stream`; *gbps receives bytes x reps / time.
int mlab_stream_read(const void* buf, size_t bytes, void* sink, void* stream, int reps, double* gbps) {
  hipStream_t st = (hipStream_t)stream;
  const long long n16 = (long long)(bytes / 16);
  const unsigned grid = 256 * 16;
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, st, (const u32x4*)buf, n16, (uint32_t*)sink);
  hipEvent_t a, b;
  hipEventCreate(&a);
  hipEventCreate(&b);
  hipEventRecord(a, st);
  for (int r = 0; r < reps; ++r)
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, st, (const u32x4*)buf, n16, (uint32_t*)sink);
  hipEventRecord(b, st);
  hipEventSynchronize(b);
  float ms = 0.f;
  hipEventElapsedTime(&ms, a, b);
  hipEventDestroy(a);
  hipEventDestroy(b);
  *gbps = (double)n16 * 16.0 * reps / (ms * 1e-3) / 1e9;
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Dense bf16 MFMA rate: 2048 workgroups of 4 waves, `iters` x 4 MFMAs each.
int mlab_mfma_peak(void* sink, void* stream, int iters, double* tflops) {
  hipStream_t st = (hipStream_t)stream;
  const unsigned grid = 2048;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(grid), dim3(256), 0, st, 16, (float*)sink);
  hipEvent_t a, b;
  hipEventCreate(&a);
  hipEventCreate(&b);
  hipEventRecord(a, st);
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(grid), dim3(256), 0, st, iters, (float*)sink);
  hipEventRecord(b, st);
  hipEventSynchronize(b);
  float ms = 0.f;
  hipEventElapsedTime(&ms, a, b);
  hipEventDestroy(a);
  hipEventDestroy(b);
  *tflops = (double)grid * 4 * iters * 4 * (2.0 * 32 * 32 * 16) / (ms * 1e-3) / 1e12;
  return hipGetLastError() == hipSuccess ? 0 : -5;
}


// LDS lane pair: LDS cycles per read instruction (a wave's cycles over its 16
// x `iters` reads, divided by the 8 waves sharing the CU's LDS) with lanes li, lj (0..63) at the same (same = 1) or different
// bank sets; op 0 ds_read_b128, 1 ds_read_b64_tr_b16.  `scratch`:
// 256 x 8 x 8 bytes of device memory, `sink` 4 bytes.  Synchronises `stream`.
int mlab_lds_pair(int op, int li, int lj, int same, int iters, void* scratch, void* sink, void* stream,
                  double* clk_per_read) {
  if (op < 0 || op > 1 || li < -1 || li > 63 || lj < -1 || lj > 63 || iters < 1) return -2;
  hipStream_t st = (hipStream_t)stream;
  unsigned long long* cyc = (unsigned long long*)scratch;
  uint32_t* sk = (uint32_t*)sink;
  if (op == 0) hipLaunchKernelGGL(lds_pair_kernel<0>, dim3(256), dim3(512), 0, st, li, lj, same, iters, cyc, sk);
  if (op == 1) hipLaunchKernelGGL(lds_pair_kernel<1>, dim3(256), dim3(512), 0, st, li, lj, same, iters, cyc, sk);
  if (hipGetLastError() != hipSuccess) return -5;
  const double c = mean_cycles(cyc, st);
  if (c < 0.0) return -5;
  *clk_per_read = c / (16.0 * iters * 8.0);
  return 0;
}

// LDS layout: LDS cycles per read (as above) of the split kernel's score-fragment (pattern
// 0) or transposed V (pattern 1) reads over rows of `lrb` bytes (a multiple of
// 16, 1024..1280), chunk-swizzled when swz.  Same buffers as mlab_lds_pair.
int mlab_lds_layout(int pattern, int lrb, int swz, int iters, void* scratch, void* sink, void* stream,
                    double* clk_per_read) {
  if (pattern < 0 || pattern > 1 || lrb < 1024 || lrb > 1280 || lrb % 16 != 0 || iters < 1) return -2;
  hipStream_t st = (hipStream_t)stream;
  unsigned long long* cyc = (unsigned long long*)scratch;
  uint32_t* sk = (uint32_t*)sink;
  if (pattern == 0) hipLaunchKernelGGL(lds_layout_kernel<0>, dim3(256), dim3(512), 0, st, lrb, swz, iters, cyc, sk);
  else hipLaunchKernelGGL(lds_layout_kernel<1>, dim3(256), dim3(512), 0, st, lrb, swz, iters, cyc, sk);
  if (hipGetLastError() != hipSuccess) return -5;
  const double c = mean_cycles(cyc, st);
  if (c < 0.0) return -5;
  *clk_per_read = c / (16.0 * iters * 8.0);
  return 0;
}

}  // extern "C"
