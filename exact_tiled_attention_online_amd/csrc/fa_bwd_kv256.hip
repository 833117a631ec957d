// fa_bwd_kv256.hip -- the key/value-block-outer backward (dK, dV) at d = 256
// without dropout (with and without the dS stores); the dropout kernels are
// in fa_bwd_kv256_drop.hip.  The kernel body is fa_bwd_kv256_body.h's: two
// waves per 32-key slice, one forming S, P^ and dV, the other dP, dS and dK,
// so a workgroup of 4 waves owns 64 keys.
#include "fa_bwd_kv256_body.h"

namespace fa {

hipError_t launch_bwd_kv256(const void* q, const void* k, const void* v, const void* dO, const float* nlse,
                            const float* ndrow, void* dk, void* dv, int BH, int N, bool causal, float scale,
                            Layouts lay, hipStream_t stream, const DropArgs* drop, DsOut ds) {
  if (drop) return launch_bwd_kv256_drop(q, k, v, dO, nlse, ndrow, dk, dv, BH, N, causal, scale, lay, stream, *drop, ds);
  const DropArgs none{};
  if (ds.buf)
    return causal ? launch_bwd256_t<true, false, true>(q, k, v, dO, nlse, ndrow, dk, dv, BH, N, scale, lay, stream, none, ds)
                  : launch_bwd256_t<false, false, true>(q, k, v, dO, nlse, ndrow, dk, dv, BH, N, scale, lay, stream, none, ds);
  return causal ? launch_bwd256_t<true, false, false>(q, k, v, dO, nlse, ndrow, dk, dv, BH, N, scale, lay, stream, none, ds)
                : launch_bwd256_t<false, false, false>(q, k, v, dO, nlse, ndrow, dk, dv, BH, N, scale, lay, stream, none, ds);
}

}  // namespace fa
