// fa_bwd_kv256_drop.hip -- the key/value-block-outer backward at d = 256 with
// dropout: both kernels of the recompute dQ method and the non-causal one of
// the hand-off (the causal hand-off kernel is built in fa_bwd_kv256.hip).  The
// kernel body is fa_bwd_kv_body.h's.  These three instantiations sit in a unit
// of their own because they are built without VGPR-form MFMA results: at the
// register limit, that form makes the compiler's AGPR-copy rewrite crash on
// them.  The form only chooses where MFMA results live, so
// the arithmetic is that of every other instantiation.
#include "fa_bwd_kv_body.h"

namespace fa {

hipError_t launch_bwd_kv256_drop(const void* q, const void* k, const void* v, const void* dO, const float* nlse,
                                 const float* ndrow, void* dk, void* dv, int BH, int N, bool causal, float scale,
                                 Layouts lay, hipStream_t stream, const DropArgs& drop, DsOut ds) {
  if (!causal && ds.buf)
    return launch_bwd_dropout_t<256, false, true>(q, k, v, dO, nlse, ndrow, dk, dv, BH, N, scale, lay, stream,
                                                  drop, ds);
  if (causal && ds.buf) return hipErrorInvalidValue;   // built in fa_bwd_kv256.hip; never routed here
  return causal ? launch_bwd_dropout_t<256, true, false>(q, k, v, dO, nlse, ndrow, dk, dv, BH, N, scale, lay,
                                                         stream, drop, DsOut{})
                : launch_bwd_dropout_t<256, false, false>(q, k, v, dO, nlse, ndrow, dk, dv, BH, N, scale, lay,
                                                          stream, drop, DsOut{});
}

}  // namespace fa
