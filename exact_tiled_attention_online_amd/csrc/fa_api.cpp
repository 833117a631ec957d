// fa_api.cpp -- the C ABI declared in include/fa.h: argument checks, workspace
// carving and the kernel sequence.  No allocation, no synchronisation.
#include "../../include/fa.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <iterator>
#include <utility>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "fa_launch.h"

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kDsSink = 4096;   // the dS buffer's sink (fa::DsOut)

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Common shape / flag checks; returns FA_OK or an error status.
int check_shape(int B, int H, int N, int d, int causal, float scale, int dtype, int layout) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID;
  if (layout != FA_LAYOUT_BHND && layout != FA_LAYOUT_BNHD) return FA_ERR_INVALID;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID;
  if (!std::isfinite(scale)) return FA_ERR_INVALID;   // any finite scale (negative and 0 included)
  if (dtype != FA_BF16 && dtype != FA_FP32) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 96 && d != 128 && d != 256) return FA_ERR_UNSUPPORTED;
  // B * H * N * d < 2^31, checked factor by factor so that no product of
  // three 31-bit sizes is formed (it would overflow a 64-bit integer)
  const long long rows = (long long)B * H;
  if (rows >= (1LL << 31) || rows * N >= (1LL << 31) || rows * N * d >= (1LL << 31)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// Dense layouts: every tensor [B,H,N,d] or [B,N,H,d]; q, o, dO and dq have
// Nq rows per head, k, v, dk and dv Nk.  Sizes have passed check_shape.
fa::RowLayout dense_rows(int H, int N, int d, int layout) {
  if (layout == FA_LAYOUT_BNHD) return fa::RowLayout{(long long)N * H * d, d, H * d};
  return fa::RowLayout{(long long)H * N * d, (long long)N * d, d};
}
fa::Layouts dense_layouts(int H, int Nq, int Nk, int d, int layout) {
  const fa::RowLayout a = dense_rows(H, Nq, d, layout), b = dense_rows(H, Nk, d, layout);
  return fa::Layouts{a, b, b, a, a, a, b, b, H};
}

// One tensor's layout from a caller's element strides st = {batch, head, row}
// (rows of d contiguous elements of esize bytes).  Rejects a negative stride,
// one that breaks the 16-byte alignment of rows, a head whose rows reach
// 2^31 bytes (the kernels address a head's rows with 32-bit byte offsets), a
// view reaching past 2^62 bytes, and, for an output, a view in which two rows
// overlap (checked by the sufficient rule: with the dimensions of more than
// one entry taken by increasing stride, each stride is at least the extent of
// everything inside it).
bool strided_rows(const long long* st, int B, int H, int N, int d, int esize, bool output, fa::RowLayout* out) {
  const long long sb = st[0], sh = st[1], sn = st[2];
  const long long unit = 16 / esize;
  for (long long x : {sb, sh, sn})
    if (x < 0 || x % unit != 0 || x > (1LL << 40)) return false;
  if ((__int128)N * sn * esize >= ((__int128)1 << 31)) return false;
  const __int128 extent = (__int128)(B - 1) * sb + (__int128)(H - 1) * sh + (__int128)(N - 1) * sn + d;
  if (extent * esize > ((__int128)1 << 62)) return false;
  if (output) {
    std::pair<long long, long long> dims[3] = {{sb, B}, {sh, H}, {sn, N}};   // (stride, entries)
    std::sort(std::begin(dims), std::end(dims));
    __int128 inner = d;
    for (const auto& dm : dims) {
      if (dm.second == 1) continue;
      if ((__int128)dm.first < inner) return false;
      inner += (__int128)(dm.second - 1) * dm.first;
    }
  }
  *out = fa::RowLayout{sb, sh, (int)sn};
  return true;
}

// Bytes of the dS hand-off buffer per (batch, head): query block i (64 rows)
// holds 2i + 2 (causal) or ceil(N/32) (otherwise) slices of 4 KB.  The buffer
// is followed by a 4 KB sink (fa::DsOut).
size_t ds_head_bytes(int N, bool causal) {
  const int nqb = (N + 63) / 64, nks = (N + 31) / 32;
  return fa::ds_block_off(causal, nqb, nks);
}

// The bytes past the two per-row statistics that a dQ method needs: the fp32
// accumulator of the atomic method, the dS buffer of the hand-off, nothing for
// the recompute.  0 with ok = false where the method does not exist for the
// arguments or the size does not fit in a size_t.
size_t region_bytes(int method, int B, int H, int N, int d, bool causal, int dtype, bool* ok) {
  *ok = true;
  const size_t BH = (size_t)B * H;
  if (method == FA_DQ_RECOMPUTE) return 0;
  if (dtype != FA_BF16) {
    *ok = false;
    return 0;
  }
  if (method == FA_DQ_ATOMIC) {
    if (d != 64 && d != 128) *ok = false;
    return *ok ? round_up(BH * N * d * sizeof(float)) : 0;
  }
  if (method == FA_DQ_HANDOFF) {
    const size_t hb = ds_head_bytes(N, causal);
    if (hb > ((size_t)1 << 62) / BH) {
      *ok = false;
      return 0;
    }
    return round_up(BH * hb) + kDsSink;
  }
  *ok = false;
  return 0;
}

struct Workspace {
  float* ndrow;   // -D per query row
  float* nlse;    // -LSE / scale per query row
  char* region;   // dQ accumulator (atomic) or dS buffer (hand-off)
  size_t bytes;   // total for the method (0: the method does not exist here)
};

Workspace carve(void* base, int B, int H, int N, int d, bool causal, int dtype, int method) {
  const size_t rows = (size_t)B * H * N;
  Workspace w{};
  char* p = static_cast<char*>(base);
  size_t off = 0;
  w.ndrow = reinterpret_cast<float*>(p + off);
  off += round_up(rows * sizeof(float));
  w.nlse = reinterpret_cast<float*>(p + off);
  off += round_up(rows * sizeof(float));
  w.region = p + off;
  bool ok = false;
  const size_t extra = region_bytes(method, B, H, N, d, causal, dtype, &ok);
  w.bytes = ok ? off + extra : 0;
  return w;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// The dQ method a backward call takes.  FA_DQ_MODE=atomic (bf16, d = 64 or
// 128, not with dropout) or FA_DQ_MODE=recompute force one, for A/B
// measurement; otherwise the hand-off when the workspace holds its buffer, and
// the recompute kernel when it does not.  The choice depends only on the
// arguments and the environment, so the three stage calls of one backward
// agree.
int dq_method(int B, int H, int N, int d, bool causal, int dtype, size_t workspace_bytes, bool dropout) {
  if (dtype != FA_BF16) return FA_DQ_RECOMPUTE;
  const char* m = std::getenv("FA_DQ_MODE");
  if (m && std::strcmp(m, "atomic") == 0 && !dropout && (d == 64 || d == 128)) return FA_DQ_ATOMIC;
  if (m && std::strcmp(m, "recompute") == 0) return FA_DQ_RECOMPUTE;
  const Workspace h = carve(nullptr, B, H, N, d, causal, dtype, FA_DQ_HANDOFF);
  return (h.bytes != 0 && workspace_bytes >= h.bytes) ? FA_DQ_HANDOFF : FA_DQ_RECOMPUTE;
}

bool workspace_ok(const void* ws, size_t bytes, int B, int H, int N, int d, bool causal, int dtype, int method) {
  const size_t need = carve(nullptr, B, H, N, d, causal, dtype, method).bytes;
  return ws && aligned(ws, kAlign) && need != 0 && bytes >= need;
}

fa::DsOut ds_out(const Workspace& w, int B, int H, int N, bool causal) {
  const size_t hb = ds_head_bytes(N, causal);
  return fa::DsOut{w.region, hb, (N + 31) / 32, w.region + round_up((size_t)B * H * hb)};
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
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (causal && Nq > Nk) return FA_ERR_INVALID;
  if (num_splits < 0 || num_splits > kMaxSplits) return FA_ERR_INVALID;
  return FA_OK;
}

// The forward and backward calls on given layouts, after every check their
// public forms share (shape, flags, pointers, alignment); the public forms
// differ only in where the layouts come from.
int fwd_core(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
             int causal, float scale, void* stream, int dtype, const fa::Layouts& L) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID;
  const int st = check_shape(B, H, N, d, causal, scale, dtype, FA_LAYOUT_BHND);
  if (st != FA_OK) return st;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == FA_BF16) return hip_status(fa::launch_fwd_bf16(q, k, v, o, lse, B * H, N, d, causal != 0, scale, L, s));
  return hip_status(fa::launch_fwd_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                       static_cast<const float*>(v), static_cast<float*>(o), lse, B * H, N, d,
                                       causal != 0, scale, L, s));
}

int pre_core(const void* o, const void* dO, const float* lse, int B, int H, int N, int d, float scale,
             void* workspace, size_t workspace_bytes, void* stream, int dtype, const fa::Layouts& L) {
  if (!o || !dO || !lse) return FA_ERR_INVALID;
  const int st = check_shape(B, H, N, d, 0, scale, dtype, FA_LAYOUT_BHND);
  if (st != FA_OK) return st;
  if (!aligned(o, 16) || !aligned(dO, 16) || !aligned(lse, 4)) return FA_ERR_INVALID;
  // the statistics sit at the same place for every method; only the atomic
  // method needs more here (its accumulator is cleared)
  const bool atomic = dq_method(B, H, N, d, false, dtype, 0, false) == FA_DQ_ATOMIC;
  const int method = atomic ? FA_DQ_ATOMIC : FA_DQ_RECOMPUTE;
  if (!workspace_ok(workspace, workspace_bytes, B, H, N, d, false, dtype, method)) return FA_ERR_WORKSPACE;
  const Workspace w = carve(workspace, B, H, N, d, false, dtype, method);
  float* dq_acc = atomic ? reinterpret_cast<float*>(w.region) : nullptr;
  return hip_status(fa::launch_bwd_pre(o, dO, lse, w.ndrow, w.nlse, dq_acc, B * H, N, d, scale, dtype == FA_FP32,
                                       L, static_cast<hipStream_t>(stream)));
}

int dkdv_core(const void* q, const void* k, const void* v, const void* dO, const float* lse, void* dk, void* dv,
              int B, int H, int N, int d, int causal, float scale, void* workspace, size_t workspace_bytes,
              void* stream, int dtype, const fa::Layouts& L) {
  if (!q || !k || !v || !dO || !lse || !dk || !dv) return FA_ERR_INVALID;
  const int st = check_shape(B, H, N, d, causal, scale, dtype, FA_LAYOUT_BHND);
  if (st != FA_OK) return st;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dO, 16) || !aligned(dk, 16) ||
      !aligned(dv, 16) || !aligned(lse, 4))
    return FA_ERR_INVALID;
  const int method = dq_method(B, H, N, d, causal != 0, dtype, workspace_bytes, false);
  if (!workspace_ok(workspace, workspace_bytes, B, H, N, d, causal != 0, dtype, method)) return FA_ERR_WORKSPACE;
  const Workspace w = carve(workspace, B, H, N, d, causal != 0, dtype, method);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == FA_FP32)
    return hip_status(fa::launch_bwd_kv_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                            static_cast<const float*>(v), static_cast<const float*>(dO), lse,
                                            w.ndrow, static_cast<float*>(dk), static_cast<float*>(dv), B * H, N,
                                            d, causal != 0, scale, L, s));
  const fa::DsOut ds = method == FA_DQ_HANDOFF ? ds_out(w, B, H, N, causal != 0) : fa::DsOut{};
  return hip_status(fa::launch_bwd_bf16(q, k, v, dO, w.nlse, w.ndrow, reinterpret_cast<float*>(w.region), dk, dv,
                                        B * H, N, d, causal != 0, scale, method == FA_DQ_ATOMIC, L, s, nullptr, ds));
}

int dq_core(const void* q, const void* k, const void* v, const void* dO, const float* lse, void* dq, int B, int H,
            int N, int d, int causal, float scale, void* workspace, size_t workspace_bytes, void* stream, int dtype,
            const fa::Layouts& L) {
  if (!q || !k || !v || !dO || !lse || !dq) return FA_ERR_INVALID;
  const int st = check_shape(B, H, N, d, causal, scale, dtype, FA_LAYOUT_BHND);
  if (st != FA_OK) return st;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dO, 16) || !aligned(dq, 16) ||
      !aligned(lse, 4))
    return FA_ERR_INVALID;
  const int method = dq_method(B, H, N, d, causal != 0, dtype, workspace_bytes, false);
  if (!workspace_ok(workspace, workspace_bytes, B, H, N, d, causal != 0, dtype, method)) return FA_ERR_WORKSPACE;
  const Workspace w = carve(workspace, B, H, N, d, causal != 0, dtype, method);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == FA_FP32)
    return hip_status(fa::launch_bwd_q_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                           static_cast<const float*>(v), static_cast<const float*>(dO), lse,
                                           w.ndrow, static_cast<float*>(dq), B * H, N, d, causal != 0, scale, L,
                                           s));
  if (method == FA_DQ_ATOMIC)
    return hip_status(fa::launch_dq_convert(reinterpret_cast<float*>(w.region), dq, B * H, N, d, scale, L, s));
  if (method == FA_DQ_HANDOFF)
    return hip_status(fa::launch_bwd_dq_ds(ds_out(w, B, H, N, causal != 0), k, dq, B * H, N, d, causal != 0, scale,
                                           L, s));
  return hip_status(fa::launch_bwd_dq(q, k, v, dO, w.nlse, w.ndrow, dq, B * H, N, d, causal != 0, scale, L, s));
}

int bwd_core(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
             void* dq, void* dk, void* dv, int B, int H, int N, int d, int causal, float scale, void* workspace,
             size_t workspace_bytes, void* stream, int dtype, const fa::Layouts& L) {
  // all checks first, so that a rejected call launches nothing
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv) return FA_ERR_INVALID;
  const int st = check_shape(B, H, N, d, causal, scale, dtype, FA_LAYOUT_BHND);
  if (st != FA_OK) return st;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dO, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4))
    return FA_ERR_INVALID;
  if (!workspace_ok(workspace, workspace_bytes, B, H, N, d, causal != 0, dtype,
                    dq_method(B, H, N, d, causal != 0, dtype, workspace_bytes, false)))
    return FA_ERR_WORKSPACE;
  int r = pre_core(o, dO, lse, B, H, N, d, scale, workspace, workspace_bytes, stream, dtype, L);
  if (r != FA_OK) return r;
  r = dkdv_core(q, k, v, dO, lse, dk, dv, B, H, N, d, causal, scale, workspace, workspace_bytes, stream, dtype, L);
  if (r != FA_OK) return r;
  return dq_core(q, k, v, dO, lse, dq, B, H, N, d, causal, scale, workspace, workspace_bytes, stream, dtype, L);
}

// Layouts of the strided calls: strides holds 3 values per tensor, for the
// tensors of `slots` (members of fa::Layouts) in that order; `outputs` marks
// the slots the call writes.  Unused slots keep the first tensor's layout.
bool strided_layouts(const long long* strides, std::initializer_list<fa::RowLayout fa::Layouts::*> slots,
                     unsigned outputs, int B, int H, int N, int d, int dtype, fa::Layouts* L) {
  if (!strides) return false;
  const int esize = dtype == FA_FP32 ? 4 : 2;
  int i = 0;
  for (auto slot : slots) {
    fa::RowLayout r{};
    if (!strided_rows(strides + 3 * i, B, H, N, d, esize, (outputs >> i) & 1u, &r)) return false;
    if (i == 0) *L = fa::Layouts{r, r, r, r, r, r, r, r, H};
    L->*slot = r;
    ++i;
  }
  return true;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
           int causal, float scale, void* stream, int dtype, int layout) {
  const int st = check_shape(B, H, N, d, causal, scale, dtype, layout);
  if (st != FA_OK) return st;
  return fwd_core(q, k, v, o, lse, B, H, N, d, causal, scale, stream, dtype, dense_layouts(H, N, N, d, layout));
}

int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                   int causal, float scale, const long long* strides, void* stream, int dtype) {
  const int st = check_shape(B, H, N, d, causal, scale, dtype, FA_LAYOUT_BHND);
  if (st != FA_OK) return st;
  fa::Layouts L{};
  if (!strided_layouts(strides, {&fa::Layouts::q, &fa::Layouts::k, &fa::Layouts::v, &fa::Layouts::o}, 0x8u, B, H,
                       N, d, dtype, &L))
    return FA_ERR_INVALID;
  return fwd_core(q, k, v, o, lse, B, H, N, d, causal, scale, stream, dtype, L);
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d, int causal, int dtype, int dq_method) {
  if (check_shape(B, H, N, d, causal, 1.f, dtype, FA_LAYOUT_BHND) != FA_OK) return 0;
  return carve(nullptr, B, H, N, d, causal != 0, dtype, dq_method).bytes;
}

int fa_bwd_dq_method(int B, int H, int N, int d, int causal, int dtype, size_t workspace_bytes, int dropout) {
  const int st = check_shape(B, H, N, d, causal, 1.f, dtype, FA_LAYOUT_BHND);
  if (st != FA_OK) return st;
  if (dropout != 0 && dropout != 1) return FA_ERR_INVALID;
  if (dropout && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  return dq_method(B, H, N, d, causal != 0, dtype, workspace_bytes, dropout != 0);
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d, int dtype) {
  if (check_shape(B, H, N, d, 0, 1.f, dtype, FA_LAYOUT_BHND) != FA_OK) return 0;
  // the recompute method's statistics, or with FA_DQ_MODE=atomic the
  // accumulator too; the hand-off buffer depends on causal (fa_bwd_workspace_size)
  return carve(nullptr, B, H, N, d, false, dtype, dq_method(B, H, N, d, false, dtype, 0, false)).bytes;
}

int fa_bwd_preprocess(const void* o, const void* dO, const float* lse, int B, int H, int N, int d,
                      float scale, void* workspace, size_t workspace_bytes, void* stream, int dtype,
                      int layout) {
  const int st = check_shape(B, H, N, d, 0, scale, dtype, layout);
  if (st != FA_OK) return st;
  return pre_core(o, dO, lse, B, H, N, d, scale, workspace, workspace_bytes, stream, dtype,
                  dense_layouts(H, N, N, d, layout));
}

int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO, const float* lse, void* dk,
                void* dv, int B, int H, int N, int d, int causal, float scale, void* workspace,
                size_t workspace_bytes, void* stream, int dtype, int layout) {
  const int st = check_shape(B, H, N, d, causal, scale, dtype, layout);
  if (st != FA_OK) return st;
  return dkdv_core(q, k, v, dO, lse, dk, dv, B, H, N, d, causal, scale, workspace, workspace_bytes, stream, dtype,
                   dense_layouts(H, N, N, d, layout));
}

int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dO, const float* lse, void* dq, int B,
              int H, int N, int d, int causal, float scale, void* workspace, size_t workspace_bytes, void* stream,
              int dtype, int layout) {
  const int st = check_shape(B, H, N, d, causal, scale, dtype, layout);
  if (st != FA_OK) return st;
  return dq_core(q, k, v, dO, lse, dq, B, H, N, d, causal, scale, workspace, workspace_bytes, stream, dtype,
                 dense_layouts(H, N, N, d, layout));
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
           void* dq, void* dk, void* dv, int B, int H, int N, int d, int causal, float scale, void* workspace,
           size_t workspace_bytes, void* stream, int dtype, int layout) {
  const int st = check_shape(B, H, N, d, causal, scale, dtype, layout);
  if (st != FA_OK) return st;
  return bwd_core(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, causal, scale, workspace, workspace_bytes, stream,
                  dtype, dense_layouts(H, N, N, d, layout));
}

int fa_bwd_strided(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                   void* dq, void* dk, void* dv, int B, int H, int N, int d, int causal, float scale,
                   const long long* strides, void* workspace, size_t workspace_bytes, void* stream, int dtype) {
  const int st = check_shape(B, H, N, d, causal, scale, dtype, FA_LAYOUT_BHND);
  if (st != FA_OK) return st;
  using L8 = fa::Layouts;
  fa::Layouts L{};
  if (!strided_layouts(strides, {&L8::q, &L8::k, &L8::v, &L8::o, &L8::g, &L8::dq, &L8::dk, &L8::dv}, 0xE0u, B, H, N,
                       d, dtype, &L))
    return FA_ERR_INVALID;
  return bwd_core(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, causal, scale, workspace, workspace_bytes, stream,
                  dtype, L);
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
  return hip_status(fa::launch_fwd_bf16(q, k, v, o, lse, B * H, N, d, causal != 0, scale,
                                        dense_layouts(H, N, N, d, layout),
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
  const int method = dq_method(B, H, N, d, causal != 0, FA_BF16, workspace_bytes, true);
  if (!workspace_ok(workspace, workspace_bytes, B, H, N, d, causal != 0, FA_BF16, method)) return FA_ERR_WORKSPACE;
  const Workspace w = carve(workspace, B, H, N, d, causal != 0, FA_BF16, method);
  const fa::Layouts lay = dense_layouts(H, N, N, d, layout);
  const fa::DropArgs dr = drop_args(drop_t, seed, offset);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const fa::DsOut ds = method == FA_DQ_HANDOFF ? ds_out(w, B, H, N, causal != 0) : fa::DsOut{};
  int r = hip_status(fa::launch_bwd_pre(o, dO, lse, w.ndrow, w.nlse, nullptr, B * H, N, d, scale, false, lay, s));
  if (r != FA_OK) return r;
  r = hip_status(fa::launch_bwd_bf16(q, k, v, dO, w.nlse, w.ndrow, nullptr, dk, dv, B * H, N, d, causal != 0,
                                     scale, false, lay, s, &dr, ds));
  if (r != FA_OK) return r;
  // the dS in the buffer already carries the mask: dQ = dS K as without dropout
  if (method == FA_DQ_HANDOFF)
    return hip_status(fa::launch_bwd_dq_ds(ds, k, dq, B * H, N, d, causal != 0, scale, lay, s));
  return hip_status(fa::launch_bwd_dq(q, k, v, dO, w.nlse, w.ndrow, dq, B * H, N, d, causal != 0, scale, lay, s,
                                      &dr));
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
               int causal, float scale, float descale_q, float descale_k, float descale_v, void* stream,
               int layout) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID;
  const int st = check_shape(B, H, N, d, causal, scale, FA_BF16, layout);
  if (st != FA_OK) return st;
  for (float x : {descale_q, descale_k, descale_v})
    if (!std::isfinite(x) || !(x > 0.f)) return FA_ERR_INVALID;
  if (!std::isfinite(scale * descale_q * descale_k)) return FA_ERR_INVALID;   // the scores' factor
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_INVALID;
  return hip_status(fa::launch_fwd_fp8(q, k, v, o, lse, B * H, N, d, causal != 0, scale, descale_q, descale_k,
                                       descale_v, dense_layouts(H, N, N, d, layout),
                                       static_cast<hipStream_t>(stream)));
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
  const fa::Layouts lay = dense_layouts(H, Nq, Nk, d, layout);
  const int r = hip_status(fa::launch_fwd_split_bf16(q, k, v, p.opart, p.lpart, B * H, Nq, Nk, d, causal != 0,
                                                     scale, p.nsplit, p.span, lay, s));
  if (r != FA_OK) return r;
  return hip_status(fa::launch_fwd_merge(p.opart, p.lpart, o, lse, B * H, Nq, d, p.nsplit, lay, s));
}

size_t fa_fwd_splitkv_fp8_workspace_bytes(int B, int H, int Nq, int Nk, int d, int num_splits) {
  if (check_split(B, H, Nq, Nk, d, 0, 1.f, num_splits, FA_BF16, FA_LAYOUT_BHND) != FA_OK) return 0;
  return split_plan(nullptr, B, H, Nq, Nk, d, num_splits, fa::kSplitBC8).bytes;
}

int fa_fwd_splitkv_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq,
                       int Nk, int d, int causal, float scale, float descale_q, float descale_k, float descale_v,
                       int num_splits, void* workspace, size_t workspace_bytes, void* stream, int layout) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID;
  const int st = check_split(B, H, Nq, Nk, d, causal, scale, num_splits, FA_BF16, layout);
  if (st != FA_OK) return st;
  for (float x : {descale_q, descale_k, descale_v})
    if (!std::isfinite(x) || !(x > 0.f)) return FA_ERR_INVALID;
  if (!std::isfinite(scale * descale_q * descale_k)) return FA_ERR_INVALID;   // the scores' factor
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_INVALID;
  if (!workspace || !aligned(workspace, kAlign) ||
      workspace_bytes < split_plan(nullptr, B, H, Nq, Nk, d, num_splits, fa::kSplitBC8).bytes)
    return FA_ERR_WORKSPACE;
  const SplitPlan p = split_plan(workspace, B, H, Nq, Nk, d, num_splits, fa::kSplitBC8);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const fa::Layouts lay = dense_layouts(H, Nq, Nk, d, layout);
  const int r = hip_status(fa::launch_fwd_split_fp8(q, k, v, p.opart, p.lpart, B * H, Nq, Nk, d, causal != 0, scale,
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
    case FA_ERR_SCRATCH: return "the call needs more than the no-allocation entry point's static scratch "
                                "(FA_SPLITKV_NOALLOC_MAX_BYTES); use fewer key ranges or the workspace form";
    default: return "unknown status";
  }
}

}  // extern "C"
