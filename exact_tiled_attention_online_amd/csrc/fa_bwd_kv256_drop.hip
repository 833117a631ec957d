// fa_bwd_kv256_drop.hip -- the key/value-block-outer backward at d = 256 with
// dropout, for the recompute dQ method (the dK/dV kernel that does not store
// dS).  The kernel body is fa_bwd_kv_body.h's.  These two instantiations sit
// in a unit of their own because they are built without VGPR-form MFMA
// results: at the register limit, that form makes the compiler's AGPR-copy
// rewrite crash on them.  The form only chooses where MFMA results live, so
// the arithmetic is that of every other instantiation.
#include "fa_bwd_kv_body.h"

namespace fa {

hipError_t launch_bwd_kv256_drop(const void* q, const void* k, const void* v, const void* dO, const float* nlse,
                                 const float* ndrow, void* dk, void* dv, int BH, int N, bool causal, float scale,
                                 Layouts lay, hipStream_t stream, const DropArgs& drop) {
  return causal ? launch_bwd_dropout_t<256, true, false>(q, k, v, dO, nlse, ndrow, dk, dv, BH, N, scale, lay,
                                                         stream, drop, DsOut{})
                : launch_bwd_dropout_t<256, false, false>(q, k, v, dO, nlse, ndrow, dk, dv, BH, N, scale, lay,
                                                          stream, drop, DsOut{});
}

}  // namespace fa
