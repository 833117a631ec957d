// fa_bwd_bf16.hip -- the key/value-block-outer backward (dK, dV; fa_bwd_kv_body.h)
// for d = 64, 96 and 128, and the dispatch over head dims (d = 256 lives in
// fa_bwd_kv256.hip, which the build compiles without VGPR-form MFMA results).
#include "fa_bwd_kv_body.h"

namespace fa {

template <bool DQA>
static hipError_t launch_bwd_kv(const void* q, const void* k, const void* v, const void* dO,
                                const float* nlse, const float* ndrow, float* dq_acc, void* dk, void* dv,
                                int BH, int N, int d, bool causal, float scale, RowLayout lay,
                                hipStream_t stream, const DropArgs* drop) {
  if (d == 128)
    return causal ? launch_bwd_bf16_t<128, true, DQA>(q, k, v, dO, nlse, ndrow, dq_acc, dk, dv, BH, N, scale, lay, stream, drop)
                  : launch_bwd_bf16_t<128, false, DQA>(q, k, v, dO, nlse, ndrow, dq_acc, dk, dv, BH, N, scale, lay, stream, drop);
  if constexpr (!DQA) {
    if (d == 96)
      return causal ? launch_bwd_bf16_t<96, true, false>(q, k, v, dO, nlse, ndrow, dq_acc, dk, dv, BH, N, scale, lay, stream, drop)
                    : launch_bwd_bf16_t<96, false, false>(q, k, v, dO, nlse, ndrow, dq_acc, dk, dv, BH, N, scale, lay, stream, drop);
    if (d == 256) return launch_bwd_kv256(q, k, v, dO, nlse, ndrow, dk, dv, BH, N, causal, scale, lay, stream, drop);
  }
  return causal ? launch_bwd_bf16_t<64, true, DQA>(q, k, v, dO, nlse, ndrow, dq_acc, dk, dv, BH, N, scale, lay, stream, drop)
                : launch_bwd_bf16_t<64, false, DQA>(q, k, v, dO, nlse, ndrow, dq_acc, dk, dv, BH, N, scale, lay, stream, drop);
}

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* dO,
                           const float* nlse, const float* ndrow, float* dq_acc, void* dk, void* dv,
                           int BH, int N, int d, bool causal, float scale, bool dq_atomic, RowLayout lay,
                           hipStream_t stream, const DropArgs* drop) {
  // the dropout backward has no atomic-dQ form (the caller never asks for it)
  if (dq_atomic && drop) return hipErrorInvalidValue;
  return dq_atomic ? launch_bwd_kv<true>(q, k, v, dO, nlse, ndrow, dq_acc, dk, dv, BH, N, d, causal, scale, lay, stream, nullptr)
                   : launch_bwd_kv<false>(q, k, v, dO, nlse, ndrow, dq_acc, dk, dv, BH, N, d, causal, scale, lay, stream, drop);
}

}  // namespace fa
