// Host stand-ins for the kernel launchers of fa_launch.h, for checking the
// C-ABI layer (fa_api.cpp) under AddressSanitizer and UndefinedBehavior-
// Sanitizer on a host without a GPU.  Each stand-in touches, in host memory,
// every byte of the workspace regions the real kernels read or write (the
// caller passes a host buffer of exactly the size the library reports as its
// workspace), so that a carving or sizing mistake in fa_api.cpp becomes an
// out-of-bounds access the sanitizer reports.  Input and output tensors are
// opaque addresses here and are never touched.
#include <cstdlib>
#include <cstring>

#include "../../exact_tiled_attention_online_amd/csrc/fa_launch.h"

namespace {
void touch(void* p, size_t bytes) {
  if (bytes) std::memset(p, 0x5a, bytes);
}
unsigned long long g_sum = 0;
void read(const void* p, size_t bytes) {
  const unsigned char* c = static_cast<const unsigned char*>(p);
  for (size_t i = 0; i < bytes; i += 64) g_sum += c[i];
  if (bytes) g_sum += c[bytes - 1];
}
bool bad(bool cond) { return cond; }
}  // namespace

namespace fa {

hipError_t launch_fwd_bf16(const void*, const void*, const void*, void*, float*, int, int, int, bool, float, Layouts,
                           hipStream_t, const DropArgs*) {
  return hipSuccess;
}
hipError_t launch_fwd_fp8(const void*, const void*, const void*, void*, float*, int, int, int d, bool, float, float,
                          float, float, Layouts, hipStream_t) {
  return bad(d != 64 && d != 96 && d != 128 && d != 256) ? hipErrorInvalidValue : hipSuccess;
}
hipError_t launch_fwd_split_bf16(const void*, const void*, const void*, float* opart, float* lpart, int BH, int Nq,
                                 int Nk, int d, bool, float, int nsplit, int span, Layouts, hipStream_t) {
  if (bad(span % kSplitBC != 0 || (long long)nsplit * span < Nk || (long long)(nsplit - 1) * span >= Nk))
    return hipErrorInvalidValue;
  touch(opart, (size_t)nsplit * BH * Nq * d * sizeof(float));
  touch(lpart, (size_t)nsplit * BH * Nq * sizeof(float));
  return hipSuccess;
}
hipError_t launch_fwd_split_fp8(const void*, const void*, const void*, float* opart, float* lpart, int BH, int Nq,
                                int Nk, int d, bool, float, float, float, float, int nsplit, int span, Layouts,
                                hipStream_t) {
  if (bad(span % kSplitBC8 != 0 || (long long)nsplit * span < Nk || (long long)(nsplit - 1) * span >= Nk ||
          (d != 64 && d != 96 && d != 128 && d != 256)))
    return hipErrorInvalidValue;
  touch(opart, (size_t)nsplit * BH * Nq * d * sizeof(float));
  touch(lpart, (size_t)nsplit * BH * Nq * sizeof(float));
  return hipSuccess;
}
hipError_t launch_fwd_merge(const float* opart, const float* lpart, void*, float*, int BH, int Nq, int d, int nsplit,
                            Layouts, hipStream_t) {
  read(opart, (size_t)nsplit * BH * Nq * d * sizeof(float));
  read(lpart, (size_t)nsplit * BH * Nq * sizeof(float));
  return hipSuccess;
}
hipError_t launch_bwd_pre(const void*, const void*, const float*, float* ndrow, float* nlse, float* dq_acc, int BH,
                          int N, int d, float, bool, Layouts, hipStream_t) {
  touch(ndrow, (size_t)BH * N * sizeof(float));
  touch(nlse, (size_t)BH * N * sizeof(float));
  if (dq_acc) touch(dq_acc, (size_t)BH * N * d * sizeof(float));
  return hipSuccess;
}
hipError_t launch_bwd_bf16(const void*, const void*, const void*, const void*, const float* nlse, const float* ndrow,
                           float* dq_acc, void*, void*, int BH, int N, int d, bool causal, float, bool dq_atomic,
                           Layouts, hipStream_t, const DropArgs* drop, DsOut ds) {
  if (dq_atomic && (drop || ds.buf)) return hipErrorInvalidValue;
  read(nlse, (size_t)BH * N * sizeof(float));
  read(ndrow, (size_t)BH * N * sizeof(float));
  if (dq_atomic) touch(dq_acc, (size_t)BH * N * d * sizeof(float));
  if (ds.buf) {
    const int nqb = (N + 63) / 64, nks = (N + 31) / 32;
    if (bad(ds.nks != nks || ds.head_bytes != ds_block_off(causal, nqb, nks))) return hipErrorInvalidValue;
    touch(ds.buf, (size_t)BH * ds.head_bytes);
    touch(ds.sink, 4096);
  }
  return hipSuccess;
}
hipError_t launch_bwd_kv256(const void*, const void*, const void*, const void*, const float*, const float*, void*,
                            void*, int, int, bool, float, Layouts, hipStream_t, const DropArgs*, DsOut) {
  return hipSuccess;   // reached only through launch_bwd_bf16 in the real library
}
hipError_t launch_bwd_dq_ds(DsOut ds, const void*, void*, int BH, int N, int, bool causal, float, Layouts,
                            hipStream_t) {
  const int nqb = (N + 63) / 64, nks = (N + 31) / 32;
  if (bad(ds.nks != nks || ds.head_bytes != ds_block_off(causal, nqb, nks))) return hipErrorInvalidValue;
  read(ds.buf, (size_t)BH * ds.head_bytes);
  return hipSuccess;
}
hipError_t launch_bwd_dq(const void*, const void*, const void*, const void*, const float* nlse, const float* ndrow,
                         void*, int BH, int N, int, bool, float, Layouts, hipStream_t, const DropArgs*) {
  read(nlse, (size_t)BH * N * sizeof(float));
  read(ndrow, (size_t)BH * N * sizeof(float));
  return hipSuccess;
}
hipError_t launch_dq_convert(const float* dq_acc, void*, int BH, int N, int d, float, Layouts, hipStream_t) {
  read(dq_acc, (size_t)BH * N * d * sizeof(float));
  return hipSuccess;
}
hipError_t launch_fwd_f32(const float*, const float*, const float*, float*, float*, int, int, int, bool, float,
                          Layouts, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_bwd_kv_f32(const float*, const float*, const float*, const float*, const float*, const float* ndrow,
                             float*, float*, int BH, int N, int, bool, float, Layouts, hipStream_t) {
  read(ndrow, (size_t)BH * N * sizeof(float));
  return hipSuccess;
}
hipError_t launch_bwd_q_f32(const float*, const float*, const float*, const float*, const float*, const float* ndrow,
                            float*, int BH, int N, int, bool, float, Layouts, hipStream_t) {
  read(ndrow, (size_t)BH * N * sizeof(float));
  return hipSuccess;
}

}  // namespace fa

// exact-size, 256-byte-aligned host buffers standing in for device workspaces
extern "C" void* host_workspace(size_t bytes) {
  void* p = nullptr;
  return posix_memalign(&p, 256, bytes ? bytes : 1) == 0 ? p : nullptr;
}
extern "C" void host_free(void* p) { free(p); }
