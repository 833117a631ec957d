// fa_fp32.hip -- fp32 path: the same tiled method in exact fp32 VALU
// arithmetic (no MFMA rounding of operands), for fp32 callers.
//
// Work split: LP lanes own one row (query row in the forward and in the dQ
// kernel, key row in the dK/dV kernel), each lane d/LP of its elements; a dot
// product is the LP partial sums combined with xor-shuffles.  LP = 2 for
// d <= 128; at d = 256, 4 in the forward and 8 in the backward kernels, so
// that a lane's slices of its rows (q and o; k, v, dk and dv; q, dO and dq)
// stay in registers.  A workgroup of 128 lanes owns 128/LP rows.  The
// streamed operand rows sit in LDS and every lane reads the same element
// (broadcast).
//
// forward   : online softmax over 32-key tiles (page
//             "flash-attention-v2-sram-tiling" (aiqz.cc), section 5), deferred
//             normalisation, ledger LSE = m + ln l.
// backward  : key-row-outer kernel for dK, dV and query-row-outer kernel for
//             dQ, both recomputing P^ = exp(S - LSE) (page
//             "flash-attention-backpropagation" (aiqz.cc), sections 数值稳定,
//             Softmax梯度, QKV梯度); no atomics.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

// lanes per row: the forward (F) and the backward kernels (B)
template <int D> constexpr int f32_lp_fwd() { return D == 256 ? 4 : 2; }
template <int D> constexpr int f32_lp_bwd() { return D == 256 ? 8 : 2; }

// One-dimensional grid: workgroup x is row block x % nrb of head x / nrb, so
// that any number of heads the interface accepts fits (a grid's second
// dimension holds at most 65535 workgroups); a workgroup owns 128/LP rows.
inline unsigned f32_grid(int BH, int N, int LP) {
  const int rows = 128 / LP;
  return (unsigned)BH * (unsigned)((N + rows - 1) / rows);
}
constexpr int F32_TILE = 32;   // streamed rows per LDS tile

template <int D>
FA_DEV void load_rows_f32(float* dst, const float* src, int row0, int nrows, int N, int tid, int rs) {
  // dst: [F32_TILE][D] floats; src rows row0.. of one head, rs elements apart
  constexpr int V4 = D / 4;
  for (int e = tid; e < F32_TILE * V4; e += 128) {
    const int r = e / V4, c4 = e % V4;
    f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
    if (r < nrows && row0 + r < N) x = reinterpret_cast<const f32x4*>(src + (size_t)(row0 + r) * rs)[c4];
    reinterpret_cast<f32x4*>(dst + r * D)[c4] = x;
  }
}

// the dot product of a row split over LP lanes: this lane's D/LP elements,
// then the partial sums of the LP lanes
template <int D, int LP>
FA_DEV float part_dot(const float* a, const float* b) {
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < D / LP; ++c) s = fmaf(a[c], b[c], s);
#pragma unroll
  for (int x = 1; x < LP; x <<= 1) s += __shfl_xor(s, x);
  return s;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(128) void fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                      const float* __restrict__ V, float* __restrict__ O,
                                                      float* __restrict__ LSE, int BH, int N, float scale,
                                                      Layouts lay) {
  constexpr int LP = f32_lp_fwd<D>(), DH = D / LP, ROWS = 128 / LP;
  __shared__ __attribute__((aligned(16))) float sk[F32_TILE * D];
  __shared__ __attribute__((aligned(16))) float sv[F32_TILE * D];
  const int tid = threadIdx.x, half = tid & (LP - 1);   // this lane's part of the row
  const int nrb = (N + ROWS - 1) / ROWS;
  const int head = blockIdx.x / nrb;
  const int row0 = (blockIdx.x - head * nrb) * ROWS;
  const int qrow = row0 + tid / LP;
  float qh[DH], oh[DH];
#pragma unroll
  for (int c = 0; c < DH; ++c) {
    qh[c] = qrow < N ? Q[lay.off(lay.q, head) + (size_t)qrow * lay.q.sn + half * DH + c] : 0.f;
    oh[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int kv_end = CAUSAL ? min(N, row0 + ROWS) : N;
  for (int t0 = 0; t0 < kv_end; t0 += F32_TILE) {
    __syncthreads();
    load_rows_f32<D>(sk, K + lay.off(lay.k, head), t0, F32_TILE, N, tid, lay.k.sn);
    load_rows_f32<D>(sv, V + lay.off(lay.v, head), t0, F32_TILE, N, tid, lay.v.sn);
    __syncthreads();
    float s[F32_TILE];
    float mx = m;
#pragma unroll
    for (int j = 0; j < F32_TILE; ++j) {
      const int kv = t0 + j;
      float x = part_dot<D, LP>(qh, sk + j * D + half * DH) * scale;
      if (kv >= N || (CAUSAL && kv > qrow)) x = -INFINITY;
      s[j] = x;
      mx = fmaxf(mx, x);
    }
    // key 0 is never masked, so mx is finite from the first tile on
    const float alpha = expf(m - mx);
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < F32_TILE; ++j) {
      s[j] = expf(s[j] - mx);
      rs += s[j];
    }
    l = l * alpha + rs;
    m = mx;
#pragma unroll
    for (int c = 0; c < DH; ++c) {
      float acc = oh[c] * alpha;
#pragma unroll
      for (int j = 0; j < F32_TILE; ++j) acc = fmaf(s[j], sv[j * D + half * DH + c], acc);
      oh[c] = acc;
    }
  }
  if (qrow < N) {
    const float inv = 1.f / l;
    float* orow = O + lay.off(lay.o, head) + (size_t)qrow * lay.o.sn + half * DH;
#pragma unroll
    for (int c = 0; c < DH; ++c) orow[c] = oh[c] * inv;
    if (half == 0) LSE[(size_t)head * N + qrow] = m + logf(l);
  }
}

// dK, dV: a lane pair per key row; query rows stream through LDS.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(128) void bwd_kv_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                         const float* __restrict__ V, const float* __restrict__ dO,
                                                         const float* __restrict__ LSE, const float* __restrict__ NDR,
                                                         float* __restrict__ dK, float* __restrict__ dV, int N,
                                                         float scale, Layouts lay) {
  constexpr int LP = f32_lp_bwd<D>(), DH = D / LP, ROWS = 128 / LP;
  __shared__ __attribute__((aligned(16))) float sq[F32_TILE * D];
  __shared__ __attribute__((aligned(16))) float sg[F32_TILE * D];
  __shared__ float sl[F32_TILE], sd[F32_TILE];
  const int tid = threadIdx.x, half = tid & (LP - 1);   // this lane's part of the row
  const int nrb = (N + ROWS - 1) / ROWS;
  const int head = blockIdx.x / nrb;
  const int row0 = (blockIdx.x - head * nrb) * ROWS;
  const int kvrow = row0 + tid / LP;
  float kh[DH], vh[DH], dkh[DH], dvh[DH];
#pragma unroll
  for (int c = 0; c < DH; ++c) {
    kh[c] = kvrow < N ? K[lay.off(lay.k, head) + (size_t)kvrow * lay.k.sn + half * DH + c] : 0.f;
    vh[c] = kvrow < N ? V[lay.off(lay.v, head) + (size_t)kvrow * lay.v.sn + half * DH + c] : 0.f;
    dkh[c] = 0.f;
    dvh[c] = 0.f;
  }
  const int q_begin = CAUSAL ? (row0 / F32_TILE) * F32_TILE : 0;
  for (int t0 = q_begin; t0 < N; t0 += F32_TILE) {
    __syncthreads();
    load_rows_f32<D>(sq, Q + lay.off(lay.q, head), t0, F32_TILE, N, tid, lay.q.sn);
    load_rows_f32<D>(sg, dO + lay.off(lay.g, head), t0, F32_TILE, N, tid, lay.g.sn);
    if (tid < F32_TILE) {
      const int q = t0 + tid;
      sl[tid] = q < N ? LSE[(size_t)head * N + q] : 0.f;
      sd[tid] = q < N ? NDR[(size_t)head * N + q] : 0.f;
    }
    __syncthreads();
    for (int j = 0; j < F32_TILE; ++j) {
      const int q = t0 + j;
      const float sc = part_dot<D, LP>(sq + j * D + half * DH, kh) * scale;
      float p = expf(sc - sl[j]);
      if (q >= N || kvrow >= N || (CAUSAL && kvrow > q)) p = 0.f;
      const float dp = part_dot<D, LP>(sg + j * D + half * DH, vh);
      const float ds = p * (dp + sd[j]);   // sd holds -D
#pragma unroll
      for (int c = 0; c < DH; ++c) {
        dvh[c] = fmaf(p, sg[j * D + half * DH + c], dvh[c]);
        dkh[c] = fmaf(ds, sq[j * D + half * DH + c], dkh[c]);
      }
    }
  }
  if (kvrow < N) {
#pragma unroll
    for (int c = 0; c < DH; ++c) {
      dK[lay.off(lay.dk, head) + (size_t)kvrow * lay.dk.sn + half * DH + c] = dkh[c] * scale;
      dV[lay.off(lay.dv, head) + (size_t)kvrow * lay.dv.sn + half * DH + c] = dvh[c];
    }
  }
}

// dQ: a lane pair per query row; key and value rows stream through LDS.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(128) void bwd_q_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                        const float* __restrict__ V, const float* __restrict__ dO,
                                                        const float* __restrict__ LSE, const float* __restrict__ NDR,
                                                        float* __restrict__ dQ, int N, float scale, Layouts lay) {
  constexpr int LP = f32_lp_bwd<D>(), DH = D / LP, ROWS = 128 / LP;
  __shared__ __attribute__((aligned(16))) float sk[F32_TILE * D];
  __shared__ __attribute__((aligned(16))) float sv[F32_TILE * D];
  const int tid = threadIdx.x, half = tid & (LP - 1);   // this lane's part of the row
  const int nrb = (N + ROWS - 1) / ROWS;
  const int head = blockIdx.x / nrb;
  const int row0 = (blockIdx.x - head * nrb) * ROWS;
  const int qrow = row0 + tid / LP;
  float qh[DH], gh[DH], dqh[DH];
#pragma unroll
  for (int c = 0; c < DH; ++c) {
    qh[c] = qrow < N ? Q[lay.off(lay.q, head) + (size_t)qrow * lay.q.sn + half * DH + c] : 0.f;
    gh[c] = qrow < N ? dO[lay.off(lay.g, head) + (size_t)qrow * lay.g.sn + half * DH + c] : 0.f;
    dqh[c] = 0.f;
  }
  const float lse = qrow < N ? LSE[(size_t)head * N + qrow] : 0.f;
  const float ndrow = qrow < N ? NDR[(size_t)head * N + qrow] : 0.f;   // -D
  const int kv_end = CAUSAL ? min(N, row0 + ROWS) : N;
  for (int t0 = 0; t0 < kv_end; t0 += F32_TILE) {
    __syncthreads();
    load_rows_f32<D>(sk, K + lay.off(lay.k, head), t0, F32_TILE, N, tid, lay.k.sn);
    load_rows_f32<D>(sv, V + lay.off(lay.v, head), t0, F32_TILE, N, tid, lay.v.sn);
    __syncthreads();
    for (int j = 0; j < F32_TILE; ++j) {
      const int kv = t0 + j;
      const float sc = part_dot<D, LP>(qh, sk + j * D + half * DH) * scale;
      float p = expf(sc - lse);
      if (qrow >= N || kv >= N || (CAUSAL && kv > qrow)) p = 0.f;
      const float dp = part_dot<D, LP>(gh, sv + j * D + half * DH);
      const float ds = p * (dp + ndrow);
#pragma unroll
      for (int c = 0; c < DH; ++c) dqh[c] = fmaf(ds, sk[j * D + half * DH + c], dqh[c]);
    }
  }
  if (qrow < N) {
    float* dqrow = dQ + lay.off(lay.dq, head) + (size_t)qrow * lay.dq.sn + half * DH;
#pragma unroll
    for (int c = 0; c < DH; ++c) dqrow[c] = dqh[c] * scale;
  }
}

template <int D, bool CAUSAL>
static hipError_t fwd_f32_t(const float* q, const float* k, const float* v, float* o, float* lse, int BH,
                            int N, float scale, Layouts lay, hipStream_t stream) {
  const dim3 grid(f32_grid(BH, N, f32_lp_fwd<D>())), block(128);
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), grid, block, 0, stream, q, k, v, o, lse, BH, N, scale, lay);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t bwd_kv_f32_t(const float* q, const float* k, const float* v, const float* dO, const float* lse,
                               const float* ndrow, float* dk, float* dv, int BH, int N, float scale,
                               Layouts lay, hipStream_t stream) {
  const dim3 grid(f32_grid(BH, N, f32_lp_bwd<D>())), block(128);
  hipLaunchKernelGGL((bwd_kv_f32_kernel<D, CAUSAL>), grid, block, 0, stream, q, k, v, dO, lse, ndrow, dk, dv, N,
                     scale, lay);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t bwd_q_f32_t(const float* q, const float* k, const float* v, const float* dO, const float* lse,
                              const float* ndrow, float* dq, int BH, int N, float scale, Layouts lay,
                              hipStream_t stream) {
  const dim3 grid(f32_grid(BH, N, f32_lp_bwd<D>())), block(128);
  hipLaunchKernelGGL((bwd_q_f32_kernel<D, CAUSAL>), grid, block, 0, stream, q, k, v, dO, lse, ndrow, dq, N, scale,
                     lay);
  return hipGetLastError();
}

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int BH, int N,
                          int d, bool causal, float scale, Layouts lay, hipStream_t stream) {
  if (d == 128)
    return causal ? fwd_f32_t<128, true>(q, k, v, o, lse, BH, N, scale, lay, stream)
                  : fwd_f32_t<128, false>(q, k, v, o, lse, BH, N, scale, lay, stream);
  if (d == 256)
    return causal ? fwd_f32_t<256, true>(q, k, v, o, lse, BH, N, scale, lay, stream)
                  : fwd_f32_t<256, false>(q, k, v, o, lse, BH, N, scale, lay, stream);
  if (d == 96)
    return causal ? fwd_f32_t<96, true>(q, k, v, o, lse, BH, N, scale, lay, stream)
                  : fwd_f32_t<96, false>(q, k, v, o, lse, BH, N, scale, lay, stream);
  return causal ? fwd_f32_t<64, true>(q, k, v, o, lse, BH, N, scale, lay, stream)
                : fwd_f32_t<64, false>(q, k, v, o, lse, BH, N, scale, lay, stream);
}

hipError_t launch_bwd_kv_f32(const float* q, const float* k, const float* v, const float* dO, const float* lse,
                             const float* ndrow, float* dk, float* dv, int BH, int N, int d, bool causal,
                             float scale, Layouts lay, hipStream_t stream) {
  if (d == 128)
    return causal ? bwd_kv_f32_t<128, true>(q, k, v, dO, lse, ndrow, dk, dv, BH, N, scale, lay, stream)
                  : bwd_kv_f32_t<128, false>(q, k, v, dO, lse, ndrow, dk, dv, BH, N, scale, lay, stream);
  if (d == 256)
    return causal ? bwd_kv_f32_t<256, true>(q, k, v, dO, lse, ndrow, dk, dv, BH, N, scale, lay, stream)
                  : bwd_kv_f32_t<256, false>(q, k, v, dO, lse, ndrow, dk, dv, BH, N, scale, lay, stream);
  if (d == 96)
    return causal ? bwd_kv_f32_t<96, true>(q, k, v, dO, lse, ndrow, dk, dv, BH, N, scale, lay, stream)
                  : bwd_kv_f32_t<96, false>(q, k, v, dO, lse, ndrow, dk, dv, BH, N, scale, lay, stream);
  return causal ? bwd_kv_f32_t<64, true>(q, k, v, dO, lse, ndrow, dk, dv, BH, N, scale, lay, stream)
                : bwd_kv_f32_t<64, false>(q, k, v, dO, lse, ndrow, dk, dv, BH, N, scale, lay, stream);
}

hipError_t launch_bwd_q_f32(const float* q, const float* k, const float* v, const float* dO, const float* lse,
                            const float* ndrow, float* dq, int BH, int N, int d, bool causal, float scale,
                            Layouts lay, hipStream_t stream) {
  if (d == 128)
    return causal ? bwd_q_f32_t<128, true>(q, k, v, dO, lse, ndrow, dq, BH, N, scale, lay, stream)
                  : bwd_q_f32_t<128, false>(q, k, v, dO, lse, ndrow, dq, BH, N, scale, lay, stream);
  if (d == 256)
    return causal ? bwd_q_f32_t<256, true>(q, k, v, dO, lse, ndrow, dq, BH, N, scale, lay, stream)
                  : bwd_q_f32_t<256, false>(q, k, v, dO, lse, ndrow, dq, BH, N, scale, lay, stream);
  if (d == 96)
    return causal ? bwd_q_f32_t<96, true>(q, k, v, dO, lse, ndrow, dq, BH, N, scale, lay, stream)
                  : bwd_q_f32_t<96, false>(q, k, v, dO, lse, ndrow, dq, BH, N, scale, lay, stream);
  return causal ? bwd_q_f32_t<64, true>(q, k, v, dO, lse, ndrow, dq, BH, N, scale, lay, stream)
                : bwd_q_f32_t<64, false>(q, k, v, dO, lse, ndrow, dq, BH, N, scale, lay, stream);
}

}  // namespace fa
