// fa_launch.h -- internal host-side launchers, one per kernel family.  Each
// enqueues on `stream` and returns hipGetLastError(); arguments have been
// validated by the C-ABI layer (fa_api.cpp) before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

// bf16 forward: O, LSE.
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                           int N, int d, bool causal, float scale, hipStream_t stream);

// Backward preprocess: ndrow = -rowsum(dO o O) (fp32), nlse = -LSE / scale,
// and, when dq_acc is not null, dq_acc = 0.  `fp32` selects the input type.
hipError_t launch_bwd_pre(const void* o, const void* dO, const float* lse, float* ndrow, float* nlse,
                          float* dq_acc, int BH, int N, int d, float scale, bool fp32, hipStream_t stream);

// bf16 key/value-block-outer backward: dK, dV written; with dq_atomic, dQ is
// also accumulated (fp32, unscaled dS K) into dq_acc with atomics.
hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* dO,
                           const float* nlse, const float* ndrow, float* dq_acc, void* dk, void* dv,
                           int BH, int N, int d, bool causal, float scale, bool dq_atomic,
                           hipStream_t stream);

// bf16 query-block-outer dQ kernel: dQ = bf16(scale * dS K), no atomics.
hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* dO, const float* nlse,
                         const float* ndrow, void* dq, int BH, int N, int d, bool causal, float scale,
                         hipStream_t stream);

// dQ = bf16(scale * dq_acc).
hipError_t launch_dq_convert(const float* dq_acc, void* dq, size_t n, float scale, hipStream_t stream);

// fp32 path (plain VALU kernels, exact fp32 arithmetic).
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int BH, int N, int d, bool causal, float scale, hipStream_t stream);
hipError_t launch_bwd_kv_f32(const float* q, const float* k, const float* v, const float* dO,
                             const float* lse, const float* ndrow, float* dk, float* dv, int BH, int N,
                             int d, bool causal, float scale, hipStream_t stream);
hipError_t launch_bwd_q_f32(const float* q, const float* k, const float* v, const float* dO,
                            const float* lse, const float* ndrow, float* dq, int BH, int N, int d,
                            bool causal, float scale, hipStream_t stream);

}  // namespace fa
