// fa_api.cpp -- the C ABI declared in include/fa.h: argument checks, workspace
// carving and the kernel sequence.  No allocation, no synchronisation.
#include "../../include/fa.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "fa_launch.h"

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Common shape / flag checks; returns FA_OK or an error status.
int check_shape(int B, int H, int N, int d, int causal, float scale, int dtype, int layout) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID;
  if (layout != FA_LAYOUT_BHND && layout != FA_LAYOUT_BNHD) return FA_ERR_INVALID;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID;
  if (dtype != FA_BF16 && dtype != FA_FP32) return FA_ERR_UNSUPPORTED;
  // d = 256: bf16 only (the fp32 kernels hold a row of q and o per lane pair)
  if (d != 64 && d != 96 && d != 128 && !(d == 256 && dtype == FA_BF16)) return FA_ERR_UNSUPPORTED;
  const long long elems = (long long)B * H * N * d;
  if (elems >= (1LL << 31)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

fa::RowLayout row_layout(int H, int layout) { return fa::RowLayout{H, layout == FA_LAYOUT_BNHD ? 1 : 0}; }

struct Workspace {
  float* ndrow;   // -D per query row
  float* nlse;    // -LSE / scale per query row
  float* dq_acc;  // bf16 only
  size_t bytes;
};

Workspace carve(void* base, int B, int H, int N, int d, int dtype) {
  const size_t rows = (size_t)B * H * N;
  Workspace w{};
  char* p = static_cast<char*>(base);
  size_t off = 0;
  w.ndrow = reinterpret_cast<float*>(p + off);
  off += round_up(rows * sizeof(float));
  w.nlse = reinterpret_cast<float*>(p + off);
  off += round_up(rows * sizeof(float));
  w.dq_acc = nullptr;
  if (dtype == FA_BF16) {
    w.dq_acc = reinterpret_cast<float*>(p + off);
    off += round_up(rows * d * sizeof(float));
  }
  w.bytes = off;
  return w;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// dQ path of the bf16 backward: the query-block-outer kernel (default), or
// fp32 atomics from the key/value-outer kernel when FA_DQ_MODE=atomic (d = 64
// and 128 only; d = 96 and 256 always take the default).
bool dq_atomic_mode(int d) {
  const char* m = std::getenv("FA_DQ_MODE");
  return (d == 64 || d == 128) && m && std::strcmp(m, "atomic") == 0;
}

bool workspace_ok(const void* ws, size_t bytes, int B, int H, int N, int d, int dtype) {
  return ws && aligned(ws, kAlign) && bytes >= carve(nullptr, B, H, N, d, dtype).bytes;
}

// Key ranges of the split forwards (tiles of 32 keys for bf16, 64 for FP8).
// num_splits = 0 lets the library choose: about kSplitTargetWGs workgroups in
// all, at least 4 tiles per range, at most kMaxAutoSplits ranges.  Ranges are
// whole tiles and none is empty.
constexpr int kMaxAutoSplits = 256;
constexpr int kMaxSplits = 1024;
constexpr long long kSplitTargetWGs = 1024;

struct SplitPlan {
  int nsplit, span;
  float* opart;
  float* lpart;
  size_t bytes;
};

SplitPlan split_plan(void* base, int B, int H, int Nq, int Nk, int d, int num_splits, int tile = fa::kSplitBC) {
  const int tiles = (Nk + tile - 1) / tile;
  long long s = num_splits;
  if (s <= 0) {
    const long long wgs = (long long)B * H * ((Nq + 31) / 32);
    s = std::min<long long>(kMaxAutoSplits, std::max<long long>(1, (kSplitTargetWGs + wgs - 1) / wgs));
    s = std::min<long long>(s, std::max(1, tiles / 4));
  }
  s = std::min<long long>(s, tiles);
  const int per = (int)((tiles + s - 1) / s);   // tiles per range
  SplitPlan p{};
  p.nsplit = (tiles + per - 1) / per;
  p.span = per * tile;
  const size_t rows = (size_t)B * H * Nq;
  char* c = static_cast<char*>(base);
  p.opart = reinterpret_cast<float*>(c);
  const size_t ob = round_up((size_t)p.nsplit * rows * d * sizeof(float));
  p.lpart = reinterpret_cast<float*>(c + ob);
  p.bytes = ob + round_up((size_t)p.nsplit * rows * sizeof(float));
  return p;
}

int check_split(int B, int H, int Nq, int Nk, int d, int causal, float scale, int num_splits, int dtype,
                int layout) {
  int st = check_shape(B, H, Nq, d, causal, scale, dtype, layout);
  if (st != FA_OK) return st;
  st = check_shape(B, H, Nk, d, causal, scale, dtype, layout);
  if (st != FA_OK) return st;
  if (dtype != FA_BF16 || d == 256) return FA_ERR_UNSUPPORTED;
  if (causal && Nq > Nk) return FA_ERR_INVALID;
  if (num_splits < 0 || num_splits > kMaxSplits) return FA_ERR_INVALID;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
           int causal, float scale, void* stream, int dtype, int layout) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID;
  const int st = check_shape(B, H, N, d, causal, scale, dtype, layout);
  if (st != FA_OK) return st;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == FA_BF16)
    return hip_status(fa::launch_fwd_bf16(q, k, v, o, lse, B * H, N, d, causal != 0, scale, row_layout(H, layout), s));
  return hip_status(fa::launch_fwd_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                       static_cast<const float*>(v), static_cast<float*>(o), lse, B * H, N, d,
                                       causal != 0, scale, row_layout(H, layout), s));
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d, int dtype) {
  if (B < 1 || H < 1 || N < 1 || (dtype != FA_BF16 && dtype != FA_FP32) ||
      (d != 64 && d != 96 && d != 128 && !(d == 256 && dtype == FA_BF16)))
    return 0;
  return carve(nullptr, B, H, N, d, dtype).bytes;
}

int fa_bwd_preprocess(const void* o, const void* dO, const float* lse, int B, int H, int N, int d,
                      float scale, void* workspace, size_t workspace_bytes, void* stream, int dtype,
                      int layout) {
  if (!o || !dO || !lse) return FA_ERR_INVALID;
  const int st = check_shape(B, H, N, d, 0, scale, dtype, layout);
  if (st != FA_OK) return st;
  if (!aligned(o, 16) || !aligned(dO, 16) || !aligned(lse, 4)) return FA_ERR_INVALID;
  if (!workspace_ok(workspace, workspace_bytes, B, H, N, d, dtype)) return FA_ERR_WORKSPACE;
  const Workspace w = carve(workspace, B, H, N, d, dtype);
  float* dq_acc = (dtype == FA_BF16 && dq_atomic_mode(d)) ? w.dq_acc : nullptr;
  return hip_status(fa::launch_bwd_pre(o, dO, lse, w.ndrow, w.nlse, dq_acc, B * H, N, d, scale,
                                       dtype == FA_FP32, row_layout(H, layout), static_cast<hipStream_t>(stream)));
}

int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO, const float* lse, void* dk,
                void* dv, int B, int H, int N, int d, int causal, float scale, void* workspace,
                size_t workspace_bytes, void* stream, int dtype, int layout) {
  if (!q || !k || !v || !dO || !lse || !dk || !dv) return FA_ERR_INVALID;
  const int st = check_shape(B, H, N, d, causal, scale, dtype, layout);
  if (st != FA_OK) return st;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dO, 16) || !aligned(dk, 16) ||
      !aligned(dv, 16) || !aligned(lse, 4))
    return FA_ERR_INVALID;
  if (!workspace_ok(workspace, workspace_bytes, B, H, N, d, dtype)) return FA_ERR_WORKSPACE;
  const Workspace w = carve(workspace, B, H, N, d, dtype);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == FA_FP32)
    return hip_status(fa::launch_bwd_kv_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                            static_cast<const float*>(v), static_cast<const float*>(dO), lse,
                                            w.ndrow, static_cast<float*>(dk), static_cast<float*>(dv), B * H, N,
                                            d, causal != 0, scale, row_layout(H, layout), s));
  return hip_status(fa::launch_bwd_bf16(q, k, v, dO, w.nlse, w.ndrow, w.dq_acc, dk, dv, B * H, N, d,
                                        causal != 0, scale, dq_atomic_mode(d), row_layout(H, layout), s));
}

int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dO, const float* lse, void* dq, int B,
              int H, int N, int d, int causal, float scale, void* workspace, size_t workspace_bytes, void* stream,
              int dtype, int layout) {
  if (!q || !k || !v || !dO || !lse || !dq) return FA_ERR_INVALID;
  const int st = check_shape(B, H, N, d, causal, scale, dtype, layout);
  if (st != FA_OK) return st;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dO, 16) || !aligned(dq, 16) ||
      !aligned(lse, 4))
    return FA_ERR_INVALID;
  if (!workspace_ok(workspace, workspace_bytes, B, H, N, d, dtype)) return FA_ERR_WORKSPACE;
  const Workspace w = carve(workspace, B, H, N, d, dtype);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == FA_FP32)
    return hip_status(fa::launch_bwd_q_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                           static_cast<const float*>(v), static_cast<const float*>(dO), lse,
                                           w.ndrow, static_cast<float*>(dq), B * H, N, d, causal != 0, scale,
                                           row_layout(H, layout), s));
  if (dq_atomic_mode(d))
    return hip_status(fa::launch_dq_convert(w.dq_acc, dq, B * H, N, d, scale, row_layout(H, layout), s));
  return hip_status(fa::launch_bwd_dq(q, k, v, dO, w.nlse, w.ndrow, dq, B * H, N, d, causal != 0, scale,
                                      row_layout(H, layout), s));
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
           void* dq, void* dk, void* dv, int B, int H, int N, int d, int causal, float scale, void* workspace,
           size_t workspace_bytes, void* stream, int dtype, int layout) {
  // all checks first, so that a rejected call launches nothing
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv) return FA_ERR_INVALID;
  const int st = check_shape(B, H, N, d, causal, scale, dtype, layout);
  if (st != FA_OK) return st;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dO, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4))
    return FA_ERR_INVALID;
  if (!workspace_ok(workspace, workspace_bytes, B, H, N, d, dtype)) return FA_ERR_WORKSPACE;
  int r = fa_bwd_preprocess(o, dO, lse, B, H, N, d, scale, workspace, workspace_bytes, stream, dtype, layout);
  if (r != FA_OK) return r;
  r = fa_bwd_dkdv(q, k, v, dO, lse, dk, dv, B, H, N, d, causal, scale, workspace, workspace_bytes, stream, dtype,
                  layout);
  if (r != FA_OK) return r;
  return fa_bwd_dq(q, k, v, dO, lse, dq, B, H, N, d, causal, scale, workspace, workspace_bytes, stream, dtype,
                   layout);
}

namespace {
fa::DropArgs drop_args(int drop_t, unsigned long long seed, unsigned offset) {
  return fa::DropArgs{(unsigned)(seed & 0xFFFFFFFFull), (unsigned)(seed >> 32), offset, (unsigned)drop_t,
                      256.f / (float)(256 - drop_t)};
}
}  // namespace

int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                   int causal, float scale, int drop_t, unsigned long long seed, unsigned offset, void* stream,
                   int layout) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID;
  const int st = check_shape(B, H, N, d, causal, scale, FA_BF16, layout);
  if (st != FA_OK) return st;
  if (drop_t < 0 || drop_t > 255) return FA_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_INVALID;
  const fa::DropArgs dr = drop_args(drop_t, seed, offset);
  return hip_status(fa::launch_fwd_bf16(q, k, v, o, lse, B * H, N, d, causal != 0, scale, row_layout(H, layout),
                                        static_cast<hipStream_t>(stream), &dr));
}

int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                   void* dq, void* dk, void* dv, int B, int H, int N, int d, int causal, float scale, int drop_t,
                   unsigned long long seed, unsigned offset, void* workspace, size_t workspace_bytes,
                   void* stream, int layout) {
  // all checks first, so that a rejected call launches nothing
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv) return FA_ERR_INVALID;
  const int st = check_shape(B, H, N, d, causal, scale, FA_BF16, layout);
  if (st != FA_OK) return st;
  if (drop_t < 0 || drop_t > 255) return FA_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dO, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4))
    return FA_ERR_INVALID;
  if (!workspace_ok(workspace, workspace_bytes, B, H, N, d, FA_BF16)) return FA_ERR_WORKSPACE;
  const Workspace w = carve(workspace, B, H, N, d, FA_BF16);
  const fa::RowLayout lay = row_layout(H, layout);
  const fa::DropArgs dr = drop_args(drop_t, seed, offset);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int r = hip_status(fa::launch_bwd_pre(o, dO, lse, w.ndrow, w.nlse, nullptr, B * H, N, d, scale, false, lay, s));
  if (r != FA_OK) return r;
  r = hip_status(fa::launch_bwd_bf16(q, k, v, dO, w.nlse, w.ndrow, nullptr, dk, dv, B * H, N, d, causal != 0,
                                     scale, false, lay, s, &dr));
  if (r != FA_OK) return r;
  return hip_status(fa::launch_bwd_dq(q, k, v, dO, w.nlse, w.ndrow, dq, B * H, N, d, causal != 0, scale, lay, s,
                                      &dr));
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
               int causal, float scale, float descale_q, float descale_k, float descale_v, void* stream,
               int layout) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID;
  const int st = check_shape(B, H, N, d, causal, scale, FA_BF16, layout);
  if (st != FA_OK) return st;
  if (d != 128) return FA_ERR_UNSUPPORTED;
  for (float x : {descale_q, descale_k, descale_v})
    if (!std::isfinite(x) || !(x > 0.f)) return FA_ERR_INVALID;
  if (!std::isfinite(scale * descale_q * descale_k) || !(scale * descale_q * descale_k > 0.f)) return FA_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_INVALID;
  return hip_status(fa::launch_fwd_fp8(q, k, v, o, lse, B * H, N, causal != 0, scale, descale_q, descale_k,
                                       descale_v, row_layout(H, layout), static_cast<hipStream_t>(stream)));
}

size_t fa_fwd_splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int num_splits) {
  if (check_split(B, H, Nq, Nk, d, 0, 1.f, num_splits, FA_BF16, FA_LAYOUT_BHND) != FA_OK) return 0;
  return split_plan(nullptr, B, H, Nq, Nk, d, num_splits).bytes;
}

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq,
                   int Nk, int d, int causal, float scale, int num_splits, void* workspace,
                   size_t workspace_bytes, void* stream, int dtype, int layout) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID;
  const int st = check_split(B, H, Nq, Nk, d, causal, scale, num_splits, dtype, layout);
  if (st != FA_OK) return st;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_INVALID;
  if (!workspace || !aligned(workspace, kAlign) ||
      workspace_bytes < split_plan(nullptr, B, H, Nq, Nk, d, num_splits).bytes)
    return FA_ERR_WORKSPACE;
  const SplitPlan p = split_plan(workspace, B, H, Nq, Nk, d, num_splits);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const fa::RowLayout lay = row_layout(H, layout);
  const int r = hip_status(fa::launch_fwd_split_bf16(q, k, v, p.opart, p.lpart, B * H, Nq, Nk, d, causal != 0,
                                                     scale, p.nsplit, p.span, lay, s));
  if (r != FA_OK) return r;
  return hip_status(fa::launch_fwd_merge(p.opart, p.lpart, o, lse, B * H, Nq, d, p.nsplit, lay, s));
}

size_t fa_fwd_splitkv_fp8_workspace_bytes(int B, int H, int Nq, int Nk, int d, int num_splits) {
  if (check_split(B, H, Nq, Nk, d, 0, 1.f, num_splits, FA_BF16, FA_LAYOUT_BHND) != FA_OK || d != 128) return 0;
  return split_plan(nullptr, B, H, Nq, Nk, d, num_splits, fa::kSplitBC8).bytes;
}

int fa_fwd_splitkv_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq,
                       int Nk, int d, int causal, float scale, float descale_q, float descale_k, float descale_v,
                       int num_splits, void* workspace, size_t workspace_bytes, void* stream, int layout) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID;
  const int st = check_split(B, H, Nq, Nk, d, causal, scale, num_splits, FA_BF16, layout);
  if (st != FA_OK) return st;
  if (d != 128) return FA_ERR_UNSUPPORTED;
  for (float x : {descale_q, descale_k, descale_v})
    if (!std::isfinite(x) || !(x > 0.f)) return FA_ERR_INVALID;
  if (!std::isfinite(scale * descale_q * descale_k) || !(scale * descale_q * descale_k > 0.f)) return FA_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_INVALID;
  if (!workspace || !aligned(workspace, kAlign) ||
      workspace_bytes < split_plan(nullptr, B, H, Nq, Nk, d, num_splits, fa::kSplitBC8).bytes)
    return FA_ERR_WORKSPACE;
  const SplitPlan p = split_plan(workspace, B, H, Nq, Nk, d, num_splits, fa::kSplitBC8);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const fa::RowLayout lay = row_layout(H, layout);
  const int r = hip_status(fa::launch_fwd_split_fp8(q, k, v, p.opart, p.lpart, B * H, Nq, Nk, causal != 0, scale,
                                                    descale_q, descale_k, descale_v, p.nsplit, p.span, lay, s));
  if (r != FA_OK) return r;
  return hip_status(fa::launch_fwd_merge(p.opart, p.lpart, o, lse, B * H, Nq, d, p.nsplit, lay, s));
}

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID: return "invalid argument (null or misaligned pointer, bad size, flag or scale)";
    case FA_ERR_UNSUPPORTED: return "unsupported head dim, dtype or size";
    case FA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case FA_ERR_HIP: return "HIP runtime reported a launch error";
    default: return "unknown status";
  }
}

}  // extern "C"
