// fa_bwd_kv256_drop.hip -- the key/value-block-outer backward at d = 256 with
// dropout (with and without the dS stores).  The kernel body is
// fa_bwd_kv256_body.h's; these instantiations sit in a unit of their own so
// that they compile in parallel with the others.
#include "fa_bwd_kv256_body.h"

namespace fa {

hipError_t launch_bwd_kv256_drop(const void* q, const void* k, const void* v, const void* dO, const float* nlse,
                                 const float* ndrow, void* dk, void* dv, int BH, int N, bool causal, float scale,
                                 Layouts lay, hipStream_t stream, const DropArgs& drop, DsOut ds) {
  if (ds.buf)
    return causal ? launch_bwd256_t<true, true, true>(q, k, v, dO, nlse, ndrow, dk, dv, BH, N, scale, lay, stream, drop, ds)
                  : launch_bwd256_t<false, true, true>(q, k, v, dO, nlse, ndrow, dk, dv, BH, N, scale, lay, stream, drop, ds);
  return causal ? launch_bwd256_t<true, true, false>(q, k, v, dO, nlse, ndrow, dk, dv, BH, N, scale, lay, stream, drop, ds)
                : launch_bwd256_t<false, true, false>(q, k, v, dO, nlse, ndrow, dk, dv, BH, N, scale, lay, stream, drop, ds);
}

}  // namespace fa
