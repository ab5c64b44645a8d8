// launch_stub.cpp -- stand-ins for the kernel launchers of libmla (the
// functions internal.h declares), so that the host half of the library
// (api.cpp) can be built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer and driven on a machine without a GPU.  Each
// stand-in records that it was reached and launches nothing.
#include "internal.h"

namespace mla {

int stub_launches = 0;

static hipError_t reached() {
  ++stub_launches;
  return hipSuccess;
}

hipError_t absorbed_attn_bf16(const AbsorbedLaunch&, hipStream_t) { return reached(); }
hipError_t absorbed_attn_fp8(const AbsorbedLaunch&, const void*, const float*, hipStream_t) { return reached(); }
hipError_t absorbed_attn_sparse(const AbsorbedLaunch&, const int32_t*, const int32_t*, int, int, hipStream_t) {
  return reached();
}
hipError_t absorbed_attn_sparse_fp8(const AbsorbedLaunch&, const void*, const float*, const int32_t*, const int32_t*,
                                    int, int, hipStream_t) {
  return reached();
}
hipError_t materialized_attn_bf16(const MaterializedLaunch&, hipStream_t) { return reached(); }
bool materialized_bf16_supported(int n, int rope, int v) {
  return (n == 128 || n == 192 || n == 256) && (rope == 0 || rope == 64) && (v == 128 || v == 256);
}
hipError_t attn_f32(const AbsorbedLaunch*, const MaterializedLaunch*, hipStream_t) { return reached(); }
hipError_t combine_materialized(const MaterializedLaunch&, mla_dtype_t, float*, hipStream_t) { return reached(); }
hipError_t combine_upproj(const AbsorbedLaunch&, mla_dtype_t, float*, hipStream_t) { return reached(); }
hipError_t quantize_latent_fp8(long long, int, int, const void*, const void*, void*, float*, hipStream_t) {
  return reached();
}
hipError_t indexer_pool(const void*, long long, const int32_t*, int, int, int, bool, int, float*, int, hipStream_t) {
  return reached();
}
hipError_t indexer_pool_fixed(const void*, long long, const int32_t*, int, int, int, int, float*, int, hipStream_t) {
  return reached();
}
hipError_t indexer_scores(float*, int, int, const float*, const int32_t*, int, int, float*, const uint16_t*, long long,
                          int, hipStream_t) {
  return reached();
}
hipError_t indexer_select(const float*, int, const int32_t*, int, int, const int32_t*, int32_t*, hipStream_t) {
  return reached();
}
hipError_t gemm_smallm(const GemmArgs&, hipStream_t) { return reached(); }
hipError_t fold_query(mla_dtype_t, int, int, int, int, const void*, const void*, void*, hipStream_t) {
  return reached();
}
hipError_t fold_query_fp8(int, int, int, int, int, const void*, const void*, const void*, void*, void*, hipStream_t) {
  return reached();
}
hipError_t materialize_kv(mla_dtype_t, long long, int, int, int, int, int, const void*, const void*, const void*,
                          const void*, void*, void*, hipStream_t) {
  return reached();
}

hipError_t scratch_address(void** out) {
  *out = reinterpret_cast<void*>(uintptr_t(1) << 20);   // a stand-in address, never dereferenced on the host
  return reached();
}

}  // namespace mla
