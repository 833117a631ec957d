// fa_bwd_kv256.hip -- the key/value-block-outer backward (dK, dV) at d = 256:
// the plain kernels (with and without the dS stores) and the causal dropout
// kernel with the dS stores; the other dropout kernels are in
// fa_bwd_kv256_drop.hip.
// The kernel body is fa_bwd_kv_body.h's; the d = 256 instantiations, the
// largest, sit in a unit of their own so that they compile in parallel with
// the others.  At d = 256 a wave holds K and V rows, half of dK and dV, and
// the S and dP tiles (256 + about 215-256 registers, no spills).  Two waves share
// each 32-key slice (one per half of d), so a workgroup of 4 waves owns 64
// keys here rather than the 128 of d <= 128.
#include "fa_bwd_kv_body.h"

namespace fa {

hipError_t launch_bwd_kv256(const void* q, const void* k, const void* v, const void* dO, const float* nlse,
                            const float* ndrow, void* dk, void* dv, int BH, int N, bool causal, float scale,
                            Layouts lay, hipStream_t stream, const DropArgs* drop, DsOut ds) {
  return causal ? launch_bwd_bf16_t<256, true, false>(q, k, v, dO, nlse, ndrow, nullptr, dk, dv, BH, N, scale, lay,
                                                      stream, drop, ds)
                : launch_bwd_bf16_t<256, false, false>(q, k, v, dO, nlse, ndrow, nullptr, dk, dv, BH, N, scale, lay,
                                                       stream, drop, ds);
}

}  // namespace fa
