// fa_bwd_bf16.hip -- the key/value-block-outer backward (dK, dV; fa_bwd_kv_body.h)
// for d = 64, 96 and 128, and the dispatch over head dims (d = 256 lives in
// fa_bwd_kv256.hip).
#include <cstdlib>
#include <cstring>

#include "fa_bwd_kv_body.h"

namespace fa {

template <bool DQA>
static hipError_t launch_bwd_kv(const void* q, const void* k, const void* v, const void* dO,
                                const float* nlse, const float* ndrow, float* dq_acc, void* dk, void* dv,
                                int BH, int N, int d, bool causal, float scale, Layouts lay,
                                hipStream_t stream, const DropArgs* drop, DsOut ds) {
  if (d == 128)
    return causal ? launch_bwd_bf16_t<128, true, DQA>(q, k, v, dO, nlse, ndrow, dq_acc, dk, dv, BH, N, scale, lay, stream, drop, ds)
                  : launch_bwd_bf16_t<128, false, DQA>(q, k, v, dO, nlse, ndrow, dq_acc, dk, dv, BH, N, scale, lay, stream, drop, ds);
  if constexpr (!DQA) {
    if (d == 96)
      return causal ? launch_bwd_bf16_t<96, true, false>(q, k, v, dO, nlse, ndrow, dq_acc, dk, dv, BH, N, scale, lay, stream, drop, ds)
                    : launch_bwd_bf16_t<96, false, false>(q, k, v, dO, nlse, ndrow, dq_acc, dk, dv, BH, N, scale, lay, stream, drop, ds);
    if (d == 256) return launch_bwd_kv256(q, k, v, dO, nlse, ndrow, dk, dv, BH, N, causal, scale, lay, stream, drop, ds);
  }
  return causal ? launch_bwd_bf16_t<64, true, DQA>(q, k, v, dO, nlse, ndrow, dq_acc, dk, dv, BH, N, scale, lay, stream, drop, ds)
                : launch_bwd_bf16_t<64, false, DQA>(q, k, v, dO, nlse, ndrow, dq_acc, dk, dv, BH, N, scale, lay, stream, drop, ds);
}

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* dO,
                           const float* nlse, const float* ndrow, float* dq_acc, void* dk, void* dv,
                           int BH, int N, int d, bool causal, float scale, bool dq_atomic, Layouts lay,
                           hipStream_t stream, const DropArgs* drop, DsOut ds) {
  // neither the dropout backward nor the hand-off has an atomic-dQ form (the
  // caller never asks for them)
  if (dq_atomic && (drop || ds.buf)) return hipErrorInvalidValue;
  // FA_KV_KERNEL=2 (read per call): the two-waves-per-SIMD kernel of
  // fa_bwd_kv2.hip at d = 128, plain and hand-off, for A/B measurement
  const char* e = std::getenv("FA_KV_KERNEL");
  const bool kv2 = e && std::strcmp(e, "2") == 0;
  if (kv2 && d == 128 && !dq_atomic && !drop)
    return launch_bwd_kv2(q, k, v, dO, nlse, ndrow, dk, dv, BH, N, causal, scale, lay, stream, ds);
  return dq_atomic ? launch_bwd_kv<true>(q, k, v, dO, nlse, ndrow, dq_acc, dk, dv, BH, N, d, causal, scale, lay, stream, nullptr, DsOut{})
                   : launch_bwd_kv<false>(q, k, v, dO, nlse, ndrow, dq_acc, dk, dv, BH, N, d, causal, scale, lay, stream, drop, ds);
}

}  // namespace fa
