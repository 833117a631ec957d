// fa_aux.hip -- the memory-bound kernels around the backward product kernel.
//
// bwd_pre: D_i = sum_c dO_ic * O_ic for every query row (page
// "flash-attention-backpropagation" (aiqz.cc), section Softmax梯度: the row
// term the softmax normalisation adds to dP), stored negated, plus the ledger
// divided by the scale, negated (-LSE / scale): the product kernels start
// their S and dP accumulators from these, so that the accumulators end as
// S - LSE/scale and dP - D.  Also the clear of the fp32 dQ accumulator (a fill
// kernel, so the whole backward can be captured in a graph).
// Each row of d elements is read by d/8 lanes with 16-byte (bf16) or 32-byte
// (fp32) loads (in a group of 8, 16 or 32 lanes), reduced across the group
// with xor-shuffles.
//
// dq_convert: dQ = bf16(scale * acc), 8 elements per thread, 16-byte stores.
//
// fwd_merge: the key ranges of the split forward joined per query row.  With
// each range's LSE_s and O_s (normalised by its own sum), m = max_s LSE_s,
// LSE = m + ln sum_s exp(LSE_s - m) and O = sum_s exp(LSE_s - LSE) O_s: the
// rule for joining partial softmax results (page
// "flash-attention-v2-sram-tiling" (aiqz.cc), quiz question 10: take the
// larger maximum and rescale each partial sum to it), with each range's sum
// expressed at its own LSE.  d/8 lanes per row, 8 elements each.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

// lanes given to one row of D elements: D/8 rounded up to a power of two (the
// cross-lane sums use xor-shuffles within that group)
template <int D>
constexpr int lanes_per_row() {
  return D / 8 <= 8 ? 8 : (D / 8 <= 16 ? 16 : 32);
}

template <int D, typename T>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                                                      const float* __restrict__ lse,
                                                      float* __restrict__ ndrow, float* __restrict__ nlse,
                                                      float* __restrict__ dq_acc, size_t rows, float inv_scale,
                                                      int N, Layouts lay) {
  constexpr int LPR = lanes_per_row<D>();   // lanes per row (D/8 of them hold 8 elements each)
  constexpr int RPB = 256 / LPR;            // rows per block
  const int tid = threadIdx.x;
  const size_t row = (size_t)blockIdx.x * RPB + tid / LPR;
  const int part = tid % LPR;
  float acc = 0.f;
  if (row < rows && part < D / 8) {
    // row = hb*N + n of the [B*H][N] statistics; the tensor row is found
    // through the layout
    const int hb = (int)(row / N), n = (int)(row - (size_t)hb * N);
    const size_t obase = lay.off(lay.o, hb) + (size_t)n * lay.o.sn + part * 8;
    const size_t gbase = lay.off(lay.g, hb) + (size_t)n * lay.g.sn + part * 8;
    if constexpr (sizeof(T) == 2) {
      const bf16x8 o8 = *reinterpret_cast<const bf16x8*>(O + obase);
      const bf16x8 g8 = *reinterpret_cast<const bf16x8*>(dO + gbase);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)o8[e], (float)g8[e], acc);
    } else {
      const f32x4* o4 = reinterpret_cast<const f32x4*>(O + obase);
      const f32x4* g4 = reinterpret_cast<const f32x4*>(dO + gbase);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x4 a = o4[h], b = g4[h];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = fmaf(a[e], b[e], acc);
      }
    }
    if (dq_acc) {
      f32x4* z = reinterpret_cast<f32x4*>(dq_acc + row * D + part * 8);   // contiguous
      z[0] = f32x4{0.f, 0.f, 0.f, 0.f};
      z[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
  if (row < rows && part == 0) {
    ndrow[row] = -acc;
    nlse[row] = -lse[row] * inv_scale;
  }
}

hipError_t launch_bwd_pre(const void* o, const void* dO, const float* lse, float* ndrow, float* nlse,
                          float* dq_acc, int BH, int N, int d, float scale, bool fp32, Layouts lay,
                          hipStream_t stream) {
  const float inv_scale = 1.f / ledger_scale(scale);   // the ledger the bf16 kernels start from
  const size_t rows = (size_t)BH * N;
  auto go = [&](auto dc, auto tc) {
    constexpr int D = decltype(dc)::value;
    using T = std::conditional_t<decltype(tc)::value == 1, float, bf16>;
    constexpr int rpb = 256 / lanes_per_row<D>();
    const dim3 grid((unsigned)((rows + rpb - 1) / rpb)), block(256);
    hipLaunchKernelGGL((bwd_pre_kernel<D, T>), grid, block, 0, stream, (const T*)o, (const T*)dO, lse, ndrow,
                       nlse, dq_acc, rows, inv_scale, N, lay);
  };
  if (fp32) {
    if (d == 128) go(IC<128>{}, IC<1>{});
    else if (d == 96) go(IC<96>{}, IC<1>{});
    else if (d == 256) go(IC<256>{}, IC<1>{});
    else go(IC<64>{}, IC<1>{});
  } else {
    if (d == 128) go(IC<128>{}, IC<0>{});
    else if (d == 96) go(IC<96>{}, IC<0>{});
    else if (d == 256) go(IC<256>{}, IC<0>{});
    else go(IC<64>{}, IC<0>{});
  }
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void dq_convert_kernel(const float* __restrict__ acc, bf16* __restrict__ dq,
                                                         size_t n8, float scale, int N, int D, Layouts lay) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  // i = (hb*N + n)*(D/8) + c8 in the contiguous accumulator
  const int c8 = (int)(i % (D / 8));
  const size_t row = i / (D / 8);
  const int hb = (int)(row / N), n = (int)(row - (size_t)hb * N);
  const size_t out = lay.off(lay.dq, hb) + (size_t)n * lay.dq.sn + 8 * c8;
  const f32x4* a = reinterpret_cast<const f32x4*>(acc) + 2 * i;
  const f32x4 x = a[0], y = a[1];
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = (bf16)(x[e] * scale);
    r[4 + e] = (bf16)(y[e] * scale);
  }
  *reinterpret_cast<bf16x8*>(dq + out) = r;
}

hipError_t launch_dq_convert(const float* dq_acc, void* dq, int BH, int N, int d, float scale, Layouts lay,
                             hipStream_t stream) {
  const size_t n8 = (size_t)BH * N * d / 8;
  const dim3 grid((unsigned)((n8 + 255) / 256)), block(256);
  hipLaunchKernelGGL(dq_convert_kernel, grid, block, 0, stream, dq_acc, (bf16*)dq, n8, scale, N, d, lay);
  return hipGetLastError();
}

template <int D>
__global__ __launch_bounds__(256) void fwd_merge_kernel(const float* __restrict__ opart,
                                                        const float* __restrict__ lpart, bf16* __restrict__ O,
                                                        float* __restrict__ LSE, int rows, int N, int nsplit,
                                                        Layouts lay) {
  constexpr int LPR = lanes_per_row<D>();   // lanes per row (D/8 of them hold 8 elements each)
  constexpr int RPB = 256 / LPR;            // rows per block
  const int tid = threadIdx.x;
  const int row = blockIdx.x * RPB + tid / LPR;
  const int part = tid % LPR;
  if (row >= rows || part >= D / 8) return;
  float m = -INFINITY;
  for (int s = 0; s < nsplit; ++s) m = fmaxf(m, lpart[(size_t)s * rows + row]);
  float wsum = 0.f, acc[8] = {};
  for (int s = 0; s < nsplit; ++s) {
    const float ls = lpart[(size_t)s * rows + row];
    // a range in which the row sees no key has LSE -inf and weight 0
    const float w = ls == -INFINITY ? 0.f : exp2_fast((ls - m) * kLog2e);
    wsum += w;
    const float4* op = reinterpret_cast<const float4*>(opart + ((size_t)s * rows + row) * D + part * 8);
    const float4 a = op[0], b = op[1];
    acc[0] = fmaf(w, a.x, acc[0]);
    acc[1] = fmaf(w, a.y, acc[1]);
    acc[2] = fmaf(w, a.z, acc[2]);
    acc[3] = fmaf(w, a.w, acc[3]);
    acc[4] = fmaf(w, b.x, acc[4]);
    acc[5] = fmaf(w, b.y, acc[5]);
    acc[6] = fmaf(w, b.z, acc[6]);
    acc[7] = fmaf(w, b.w, acc[7]);
  }
  const float inv = 1.f / wsum;
  const int hb = row / N, n = row - hb * N;
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)(acc[e] * inv);
  *reinterpret_cast<bf16x8*>(O + lay.off(lay.o, hb) + (size_t)n * lay.o.sn + part * 8) = r;
  if (part == 0) LSE[row] = m + log2_fast(wsum) * kLn2;
}

hipError_t launch_fwd_merge(const float* opart, const float* lpart, void* o, float* lse, int BH, int Nq,
                            int d, int nsplit, Layouts lay, hipStream_t stream) {
  const int rows = BH * Nq;
  auto go = [&](auto dc) {
    constexpr int D = decltype(dc)::value;
    constexpr int rpb = 256 / lanes_per_row<D>();
    const dim3 grid((unsigned)((rows + rpb - 1) / rpb)), block(256);
    hipLaunchKernelGGL((fwd_merge_kernel<D>), grid, block, 0, stream, opart, lpart, (bf16*)o, lse, rows, Nq,
                       nsplit, lay);
  };
  if (d == 128) go(IC<128>{});
  else if (d == 256) go(IC<256>{});
  else if (d == 96) go(IC<96>{});
  else go(IC<64>{});
  return hipGetLastError();
}

}  // namespace fa
