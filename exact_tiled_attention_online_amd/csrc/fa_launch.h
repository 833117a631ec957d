// fa_launch.h -- internal host-side launchers, one per kernel family.  Each
// enqueues on `stream` and returns hipGetLastError(); arguments have been
// validated by the C-ABI layer (fa_api.cpp) before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>

namespace fa {

// Where the rows of one tensor sit: element c of row n of head h in batch b
// is b*sb + h*sh + n*sn + c elements past the tensor's base (the d elements
// of a row are contiguous).  hb is the flattened index b*H + h.  The dense
// [B,H,N,d] and [B,N,H,d] orders are two choices of the strides; a view into
// a packed projection buffer (q, k, v as slices of one [B,N,3,H,d] tensor) is
// another.
struct RowLayout {
  long long sb, sh;   // batch and head strides (elements)
  int sn;             // row stride (elements)
};

// The layouts of every tensor of one call (g: dO); each kernel reads those of
// the tensors it touches.  H is common to all, so a kernel splits hb once.
struct Layouts {
  RowLayout q, k, v, o, g, dq, dk, dv;
  int H;   // heads per batch
  // 1 for a negative scale in the bf16 and FP8 forwards: they flip the sign
  // of their Q operand and run the softmax with softmax_scale(scale) > 0.  Set
  // by the forward launchers from the scale they are given.
  int qk_neg = 0;
  __host__ __device__ __forceinline__ size_t off(const RowLayout& t, int hb) const {
    const int b = hb / H, h = hb - b * H;
    return (size_t)((long long)b * t.sb + (long long)h * t.sh);
  }
};

// The scale the softmax of the bf16 and FP8 forwards runs with: |scale|, at
// least 2^-100.  They take the row maximum of raw dot products q.k, which needs
// a positive scale; the sign of a negative one goes into Q (Layouts::qk_neg).
// Below 2^-100 in magnitude (0 included) every score of a row is the same to
// fp32 rounding (|scale * q.k| < 2^-100 times the largest dot product), as it
// is with 2^-100.
inline float softmax_scale(float scale) { return fmaxf(fabsf(scale), 0x1p-100f); }

// The scale of the backward's ledger -LSE/scale and of its recompute
// P^ = 2^(scale log2(e) (q.k - LSE/scale)), which holds for either sign: the
// caller's scale, or 2^-100 below 2^-100 in magnitude, where every recomputed
// probability of a row is e^-LSE to fp32 rounding and the ledger must stay
// finite.  dQ and dK keep the caller's scale.
inline float ledger_scale(float scale) { return fabsf(scale) >= 0x1p-100f ? scale : 0x1p-100f; }

// Arguments of the forward kernels' split-key-range mode (unused otherwise).
struct SplitArgs {
  int Nk;         // key/value rows per head
  int off;        // causal offset: query row i sits at key position i + off (off = Nk - Nq)
  int nsplit;     // key ranges per head
  int span;       // keys per range, a multiple of the kernel's tile
  float* opart;   // [nsplit][BH][N][D]: each range's O, normalised by its own l
  float* lpart;   // [nsplit][BH][N]: each range's LSE, -inf where a row sees no key of it
};

// Attention dropout (inverted, on the normalised probabilities): score
// (query i, key j) of head bh is kept iff byte j%4 of word i%4 of
// Philox4x32-10(counter (j/4, i/4, bh, offset), key (k0, k1)) is >= thresh;
// kept probabilities are multiplied by keep_scale = 256 / (256 - thresh).
struct DropArgs {
  unsigned k0, k1;    // Philox key: the seed's low and high 32 bits
  unsigned offset;    // counter word 3
  unsigned thresh;    // t in 0..255: drop probability t / 256
  float keep_scale;   // 256 / (256 - t)
};

// dS hand-off buffer, written by the key/value-outer backward kernel and
// streamed by the dS K kernel.  Unit: a 1 KB micro-tile, dS of 32 keys x 16
// queries as the 64 lanes of a wave hold it after the elementwise step: lane
// key + 32h holds 16 bytes, queries 16st + 4h + 0..3 then 16st + 8 + 4h + 0..3
// (st: the 16-query group within a 64-query block).  Per (batch, head), query
// block i (64 rows) holds its 32-key slices ks in order, 4 KB each (micro-tiles
// st = 0..3): causal slices 0..2i+1 (those reaching the diagonal; the last
// block may leave its last slot unused), otherwise slices 0..nks-1.  Entries of
// masked (query, key) pairs inside a stored slice hold 0.
struct DsOut {
  char* buf;          // the buffer (null: no hand-off)
  size_t head_bytes;  // bytes per (batch, head): ds_block_off(causal, nqb, nks)
  int nks;            // 32-key slices per head, ceil(N / 32)
  char* sink;         // 4 KB that absorb the stores of waves with no dS to store
};
__host__ __device__ __forceinline__ size_t ds_block_off(bool causal, int i, int nks) {
  return causal ? (size_t)i * (size_t)(i + 1) * 4096u : (size_t)i * (size_t)nks * 4096u;
}

// bf16 forward: O, LSE; with `drop`, O uses the dropped probabilities (LSE
// does not change).
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                           int N, int d, bool causal, float scale, Layouts lay, hipStream_t stream,
                           const DropArgs* drop = nullptr);

// FP8 (e4m3fn) forward, d = 64, 96, 128 or 256: O (bf16) and LSE for Q = dq * Q8,
// K = dk * K8, V = dv * V8.
hipError_t launch_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N, int d,
                          bool causal, float scale, float dq, float dk, float dv, Layouts lay,
                          hipStream_t stream);

// Split-key-range bf16 forward (Nq queries against Nk >= Nq keys): the keys
// of each head are cut into nsplit ranges of `span` keys (a multiple of
// kSplitBC); writes each range's O (fp32, normalised by its own sum) to opart
// [nsplit][BH][Nq][d] and its LSE to lpart [nsplit][BH][Nq].
constexpr int kSplitBC = 32;
hipError_t launch_fwd_split_bf16(const void* q, const void* k, const void* v, float* opart, float* lpart,
                                 int BH, int Nq, int Nk, int d, bool causal, float scale, int nsplit,
                                 int span, Layouts lay, hipStream_t stream);

// The same for FP8 (e4m3fn) q, k, v with per-tensor descales, d = 64, 96, 128
// or 256; ranges are whole kSplitBC8-key tiles.
constexpr int kSplitBC8 = 64;
hipError_t launch_fwd_split_fp8(const void* q, const void* k, const void* v, float* opart, float* lpart,
                                int BH, int Nq, int Nk, int d, bool causal, float scale, float dq, float dk, float dv,
                                int nsplit, int span, Layouts lay, hipStream_t stream);

// Combines the ranges of the split forward: O (bf16, layout lay.o) and LSE.
hipError_t launch_fwd_merge(const float* opart, const float* lpart, void* o, float* lse, int BH, int Nq,
                            int d, int nsplit, Layouts lay, hipStream_t stream);

// Backward preprocess: ndrow = -rowsum(dO o O) (fp32), nlse = -LSE / scale,
// and, when dq_acc is not null, dq_acc = 0.  `fp32` selects the input type.
hipError_t launch_bwd_pre(const void* o, const void* dO, const float* lse, float* ndrow, float* nlse,
                          float* dq_acc, int BH, int N, int d, float scale, bool fp32, Layouts lay,
                          hipStream_t stream);

// bf16 key/value-block-outer backward: dK, dV written; with dq_atomic, dQ is
// also accumulated (fp32, unscaled dS K) into dq_acc with atomics; with a
// non-null ds.buf (not with dq_atomic), every computed dS block is stored to
// the hand-off buffer.  With `drop` (only without dq_atomic), the gradients of
// the dropout forward.
hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* dO,
                           const float* nlse, const float* ndrow, float* dq_acc, void* dk, void* dv,
                           int BH, int N, int d, bool causal, float scale, bool dq_atomic, Layouts lay,
                           hipStream_t stream, const DropArgs* drop = nullptr, DsOut ds = DsOut{});

// The same at d = 256 (fa_bwd_kv256_body.h: two waves per 32-key slice);
// plain, with the dS stores of the hand-off method and with dropout.  It has
// no atomic-dQ form.  Dropout is passed on to launch_bwd_kv256_drop.
hipError_t launch_bwd_kv256(const void* q, const void* k, const void* v, const void* dO, const float* nlse,
                            const float* ndrow, void* dk, void* dv, int BH, int N, bool causal, float scale,
                            Layouts lay, hipStream_t stream, const DropArgs* drop, DsOut ds);

// d = 256 with dropout (the same kernel body, instantiated in a unit of its
// own so that it compiles in parallel).  ds.buf selects the form with the dS
// stores as in launch_bwd_bf16.
hipError_t launch_bwd_kv256_drop(const void* q, const void* k, const void* v, const void* dO, const float* nlse,
                                 const float* ndrow, void* dk, void* dv, int BH, int N, bool causal, float scale,
                                 Layouts lay, hipStream_t stream, const DropArgs& drop, DsOut ds);

// d = 128, without dropout or the atomic dQ: the key/value-outer kernel with
// two waves per SIMD (fa_bwd_kv2.hip); with ds.buf, also storing dS.
hipError_t launch_bwd_kv2(const void* q, const void* k, const void* v, const void* dO, const float* nlse,
                          const float* ndrow, void* dk, void* dv, int BH, int N, bool causal, float scale,
                          Layouts lay, hipStream_t stream, DsOut ds);

// dQ = bf16(scale * dS K) from the hand-off buffer (query-block outer, no
// recompute, no atomics).
hipError_t launch_bwd_dq_ds(DsOut ds, const void* k, void* dq, int BH, int N, int d, bool causal, float scale,
                            Layouts lay, hipStream_t stream);

// bf16 query-block-outer dQ kernel: dQ = bf16(scale * dS K), no atomics;
// with `drop`, the dQ of the dropout forward.
hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* dO, const float* nlse,
                         const float* ndrow, void* dq, int BH, int N, int d, bool causal, float scale,
                         Layouts lay, hipStream_t stream, const DropArgs* drop = nullptr);

// dQ = bf16(scale * dq_acc); dq_acc is contiguous [B*H][N][d], dq in layout lay.dq.
hipError_t launch_dq_convert(const float* dq_acc, void* dq, int BH, int N, int d, float scale, Layouts lay,
                             hipStream_t stream);

// fp32 path (plain VALU kernels, exact fp32 arithmetic).
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int BH, int N, int d, bool causal, float scale, Layouts lay, hipStream_t stream);
hipError_t launch_bwd_kv_f32(const float* q, const float* k, const float* v, const float* dO,
                             const float* lse, const float* ndrow, float* dk, float* dv, int BH, int N,
                             int d, bool causal, float scale, Layouts lay, hipStream_t stream);
hipError_t launch_bwd_q_f32(const float* q, const float* k, const float* v, const float* dO,
                            const float* lse, const float* ndrow, float* dq, int BH, int N, int d,
                            bool causal, float scale, Layouts lay, hipStream_t stream);

}  // namespace fa
