// internal.h -- launch descriptors shared between the C ABI layer (api.cpp)
// and the kernel files (attn.hip, gemm.hip, quant.hip, indexer.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

enum mla_dtype_t { kF32 = 0, kBF16 = 1 };

constexpr int kNumCUs = 256;   // MI355X compute units (launch planning)

// The E4M3 query block of the fp8 route: for each sequence, its L H query rows
// (row l H + h) in tiles of 32, each tile kQ8TileBytes laid out for the B
// operand of the fp8 score MFMA (16x16x128; lane l = row 16 rb + l % 16 over
// k = 128 ks + 16 (l / 16) .. + 15 (half 0) and 128 ks + 64 + 16 (l / 16) ..
// (half 1)):
//   latent codes   16 bytes at 16 ((2 (4 rb + ks) + half) 64 + l)
//   rope codes     the rope step's half 0 at kQ8RopeOff + 16 (64 rb + l)
//                  (64 values: lane groups 0..3; half 1 is zero)
//   scales         E8M0 byte of step ks at kQ8ScaleOff + 4 (64 (2 rb + ks / 4) + l)
//                  + ks % 4; lane group G holds the scale of the step's 32-wide
//                  block G (2^0 in the rope step's zero groups 2, 3)
// A block's scale 2^e is the smallest with every |q| <= 448 x 2^e; its codes
// are those of q / 2^e (nearest, ties to even).
constexpr int kQ8TileBytes = 19456, kQ8RopeOff = 16384, kQ8ScaleOff = 18432;

// Split-KV launch plan.  Sequence b is cut into ceil(Kv_b / chunk) splits;
// work item = (split, head slot, row tile).
struct SplitPlan {
  int chunk;       // positions per split, multiple of 64
  int n_splits;    // total splits over all sequences
  int row_tiles;   // ceil(rows per head slot / 64)
  int head_slots;  // absorbed: 1; materialised: H
  int n_items;     // n_splits * head_slots * row_tiles
  size_t ws_o_bytes, ws_ml_floats;   // partial O: bf16 on the absorbed bf16 route, float32 otherwise
  size_t ws_bytes;
};

struct AbsorbedLaunch {
  int r, rope, v_dim, H, B, L;
  const void* q_lat; const void* q_pe; const void* c_kv; const void* k_pe; const void* w_uv;
  const int32_t* off_dev;
  int off0, kv1;   // B == 1: the sequence's start and length (from the host offsets)
  float scale;
  void* ws_o; float* ws_ml;
  const void* q8;   // fp8 route: the fold's E4M3 query block (null: the split kernel quantises q_lat, q_pe)
  SplitPlan plan;
};

struct MaterializedLaunch {
  int n, rope, v_dim, H, B, L;
  const void* q_nope; const void* q_pe; const void* k; const void* v;
  const int32_t* off_dev;
  int off0, kv1;   // B == 1: the sequence's start and length (from the host offsets)
  float scale;
  void* ws_o; float* ws_ml;
  SplitPlan plan;
};

// attn.hip
hipError_t absorbed_attn_bf16(const AbsorbedLaunch& q, hipStream_t st);
hipError_t absorbed_attn_fp8(const AbsorbedLaunch& q, const void* codes, const float* scales, hipStream_t st);
hipError_t absorbed_attn_sparse(const AbsorbedLaunch& q, const int32_t* sel, const int32_t* koff_dev, int koff0,
                                int kvt1, hipStream_t st);
hipError_t absorbed_attn_sparse_fp8(const AbsorbedLaunch& q, const void* codes, const float* scales,
                                    const int32_t* sel, const int32_t* koff_dev, int koff0, int kvt1, hipStream_t st);
hipError_t materialized_attn_bf16(const MaterializedLaunch& q, hipStream_t st);
bool materialized_bf16_supported(int n, int rope, int v);
hipError_t attn_f32(const AbsorbedLaunch* qa, const MaterializedLaunch* qm, hipStream_t st);
hipError_t combine_materialized(const MaterializedLaunch& q, mla_dtype_t dt, float* out, hipStream_t st);
hipError_t combine_upproj(const AbsorbedLaunch& q, mla_dtype_t dt, float* out, hipStream_t st);

// quant.hip
hipError_t quantize_latent_fp8(long long T, int r, int rope, const void* c_kv, const void* k_pe, void* codes,
                               float* scales, hipStream_t st);

// indexer.hip
hipError_t indexer_pool(const void* keys, long long ld, const int32_t* off_dev, int B, int d, int S, bool full,
                        int wmax, float* pooled, int cap, hipStream_t st);
// the fixed-capacity step: P (8 or 16) windows per sequence, real updates then fillers
hipError_t indexer_pool_fixed(const void* keys, long long ld, const int32_t* off_dev, int B, int d, int S, int P,
                              float* pooled, int cap, hipStream_t st);
// tail_keys != null: the launch also pools the windows from floor((Kv - tail_S) / 4)
// on from those key rows (row stride tail_ld elements) before scoring them
hipError_t indexer_scores(float* pooled, int cap, int d, const float* q, const int32_t* off_dev, int B, int wmax,
                          float* scores, const uint16_t* tail_keys, long long tail_ld, int tail_S, hipStream_t st);
hipError_t indexer_select(const float* scores, int cap, const int32_t* off_dev, int B, int budget,
                          const int32_t* sel_off_dev, int32_t* sel, hipStream_t st);

// noalloc.hip: the device address of the static scratch array on the current
// device (looked up once per device; thread-safe).
constexpr size_t kScratchBytes = size_t(32) << 20;
hipError_t scratch_address(void** out);

// gemm.hip
struct GemmArgs {
  const uint16_t* A; long long a_row, a_head;   // element strides of A rows / heads
  const uint16_t* W;                            // [H][K][N]
  uint16_t* C; long long c_row, c_head;         // C may be null with q8 (codes only)
  int M, K, N, H;
  int n_items;
  // fold for the fp8 route: the E4M3 query blocks of C's rows and of q_pe
  uint8_t* q8;            // B x row_tiles blocks of kQ8TileBytes
  const uint16_t* q_pe;   // [B, L, H, rope]
  int L, rope, row_tiles;
};
hipError_t gemm_smallm(const GemmArgs& a, hipStream_t st);
hipError_t fold_query(mla_dtype_t dt, int rows, int H, int n, int r, const void* q_nope, const void* w_uk,
                      void* q_lat, hipStream_t st);
hipError_t fold_query_fp8(int B, int L, int H, int n, int rope, const void* q_nope, const void* w_uk,
                          const void* q_pe, void* q_lat, void* q8, hipStream_t st);
hipError_t materialize_kv(mla_dtype_t dt, long long T, int H, int r, int n, int v, int rope, const void* c_kv,
                          const void* k_pe, const void* w_uk, const void* w_uv, void* k, void* vout,
                          hipStream_t st);

}  // namespace mla
