// fa_bwd_bf16.hip -- backward kernel, bf16 inputs/outputs, fp32 accumulation.
//
// Key/value-block outer, query-block inner (page
// "flash-attention-backpropagation" (aiqz.cc), section QKV梯度): one
// workgroup (4 waves) owns BC = 128 key/value rows of one (batch, head), each
// wave 32 of them, and walks the query blocks of BR = 64 rows.  dK and dV of
// the wave's rows stay in registers for the whole walk.  Per query block and
// wave, one recompute of P^ feeds all three gradients (page "gsyq.cn
// news/1372000", 踩坑二: recomputing P once per pair of blocks):
//   S  = Q_i K_w^T                 MFMA, A = Q rows (LDS), B = K_w (registers)
//   dP = dO_i V_w^T                MFMA, A = dO rows (LDS), B = V_w (registers)
//   P^ = 2^(c*S - LSE2)            recompute from the ledger (section 数值稳定)
//   dS = P^ o (dP - D)             (section Softmax梯度)
//   dV_w += P^T dO_i               MFMA, A = P^T from the S accumulators,
//                                  B = dO through transposing LDS reads
//   dK_w += dS^T Q_i               MFMA, same shape with dS and Q
//   dQ_i += dS K                   dS goes through LDS (it is needed with the
//                                  query index across lanes); each wave takes a
//                                  32-column slice of d with K^T held in
//                                  registers; fp32 atomics into an accumulator.
// The accumulators hold fp32 and are converted once at write-back (page
// "gsyq.cn news/1372000", 踩坑三).  scale is applied to dK here and to dQ by
// the conversion kernel.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

// dS tile in LDS: [128 key rows][64 query cols] bf16, 128-byte rows of 16
// eight-byte slots; slot a of row r lives at a ^ (4*(r%4) + (r/4)%4).  The
// 8-byte writes of 16 consecutive rows at one slot, and the transposing reads
// of 4 consecutive rows x 4 consecutive slots, both touch 16 distinct slots.
FA_DEV int ds_off(int row, int col) {
  const int slot = (col >> 2) ^ (((row & 3) << 2) | ((row >> 2) & 3));
  return row * 128 + (slot << 3) + ((col & 3) << 1);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE2, const float* __restrict__ DR,
    float* __restrict__ dQacc, bf16* __restrict__ dK, bf16* __restrict__ dV, int BH, int N, int nqb,
    float scale, float c) {
  constexpr int BC = 128, BR = 64;
  constexpr int ROWB = D * 2, CH = D / 8, KS = D / 16, DT = D / 32;
  constexpr int QTB = BR * ROWB;          // bytes of one Q or dO tile
  constexpr int LPT = BR * CH / 256;      // 16-byte loads per thread per tile
  constexpr int NQT = (D == 128) ? 2 : 1; // query tiles of dQ per wave

  __shared__ __attribute__((aligned(16))) char sQ[2][QTB];
  __shared__ __attribute__((aligned(16))) char sG[2][QTB];   // dO
  __shared__ __attribute__((aligned(16))) float sL[2][BR];   // LSE * log2 e
  __shared__ __attribute__((aligned(16))) float sD[2][BR];   // D
  __shared__ __attribute__((aligned(16))) char sS[BC * BR * 2];  // dS, [key][query]
  __shared__ __attribute__((aligned(16))) char sK[BC * ROWB];    // K block (start) / output staging

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5, g = lane >> 4;
  const int bid = blockIdx.x;
  const int head = bid % BH;
  const int kb = bid / BH;                 // ascending key block = descending causal work
  const size_t hoff = (size_t)head * N * D;
  const bf16* Qh = Q + hoff;
  const bf16* Kh = K + hoff;
  const bf16* Vh = V + hoff;
  const bf16* Gh = dO + hoff;
  const float* Lh = LSE2 + (size_t)head * N;
  const float* Dh = DR + (size_t)head * N;
  float* dQh = dQacc + hoff;

  const int kv0 = kb * BC;
  const int kvw = kv0 + 32 * wave;         // first key row of this wave
  const int kvrow = kvw + l32;             // key row of this lane in the S accumulators

  // ---- K block into LDS, then the register operands -----------------------
  {
    constexpr int KPT = BC * CH / 256;
#pragma unroll
    for (int p = 0; p < KPT; ++p) {
      const int ci = p * 256 + tid;
      const int row = ci / CH, ch = ci % CH;
      const int kv = kv0 + row;
      u32x4 x = u32x4{0, 0, 0, 0};
      if (kv < N) x = *reinterpret_cast<const u32x4*>(Kh + (size_t)kv * D + ch * 8);
      *reinterpret_cast<u32x4*>(&sK[tile_off<ROWB>(row, ch)]) = x;
    }
  }
  // K_w, V_w as B operands of S = Q K^T, dP = dO V^T: lane (n = key l32, h),
  // registers d = 16*s + 8*h + r.
  bf16x8 kf[KS], vf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (kvrow < N) {
      kf[s] = *reinterpret_cast<const bf16x8*>(Kh + (size_t)kvrow * D + 16 * s + 8 * h);
      vf[s] = *reinterpret_cast<const bf16x8*>(Vh + (size_t)kvrow * D + 16 * s + 8 * h);
    } else {
      kf[s] = bf16x8{};
      vf[s] = bf16x8{};
    }
  }
  __syncthreads();
  // K^T slice as the B operand of dQ = dS K: lane (n = d col 32*dsl + l32, h),
  // registers = key rows 16*s + 8*h + r of the block.
  const int dsl = (D == 128) ? wave : (wave & 1);
  const int mt0 = (D == 128) ? 0 : (wave >> 1);
  bf16x8 ktf[BC / 16];
#pragma unroll
  for (int s = 0; s < BC / 16; ++s)
    ktf[s] = tr_operand<ROWB>(sK, 16 * s + 8 * h, 16 * s + 8 * h + 4, 32 * dsl + 16 * (g & 1), lane);

  const int i_begin = CAUSAL ? (kv0 / BR) : 0;

  u32x4 stQ[LPT], stG[LPT];
  float stL = 0.f;
  auto gload = [&](int i) {
#pragma unroll
    for (int p = 0; p < LPT; ++p) {
      const int ci = p * 256 + tid;
      const int row = ci / CH, ch = ci % CH;
      const int q = i * BR + row;
      if (q < N) {
        stQ[p] = *reinterpret_cast<const u32x4*>(Qh + (size_t)q * D + ch * 8);
        stG[p] = *reinterpret_cast<const u32x4*>(Gh + (size_t)q * D + ch * 8);
      } else {
        stQ[p] = u32x4{0, 0, 0, 0};
        stG[p] = u32x4{0, 0, 0, 0};
      }
    }
    if (tid < 2 * BR) {
      const int q = i * BR + (tid & (BR - 1));
      stL = 0.f;
      if (q < N) stL = (tid < BR) ? Lh[q] : Dh[q];
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int p = 0; p < LPT; ++p) {
      const int ci = p * 256 + tid;
      const int row = ci / CH, ch = ci % CH;
      const int off = tile_off<ROWB>(row, ch);
      *reinterpret_cast<u32x4*>(&sQ[buf][off]) = stQ[p];
      *reinterpret_cast<u32x4*>(&sG[buf][off]) = stG[p];
    }
    if (tid < BR)
      sL[buf][tid] = stL;
    else if (tid < 2 * BR)
      sD[buf][tid - BR] = stL;
  };

  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) {
    dk[t] = f32x16{};
    dv[t] = f32x16{};
  }

  if (i_begin < nqb) {
    gload(i_begin);
    swrite(0);
  }
  __syncthreads();

  for (int i = i_begin; i < nqb; ++i) {
    const int buf = (i - i_begin) & 1;
    if (i + 1 < nqb) gload(i + 1);
    const int qb0 = i * BR;
    const char* Qt = sQ[buf];
    const char* Gt = sG[buf];
    // this wave's keys are all later than all queries of the block: P^ = 0
    const bool skip = (kvw >= N) || (CAUSAL && qb0 + BR - 1 < kvw);
    if (!skip) {
      f32x16 s[2] = {f32x16{}, f32x16{}};
      f32x16 dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int off = tile_off<ROWB>(32 * t + l32, 2 * ks + h);
          s[t] = mfma32(lds_read_b128(Qt, off), kf[ks], s[t]);
          dp[t] = mfma32(lds_read_b128(Gt, off), vf[ks], dp[t]);
        }
      }
      // accumulator r of tile t: query qb0 + 32t + 8*(r/4) + 4h + r%4, key kvrow
      const bool need_mask = (CAUSAL && qb0 < kvw + 31) || (qb0 + BR > N) || (kvw + 32 > N);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int ql = 32 * t + 8 * i4 + 4 * h;
          const f32x4 L4 = *reinterpret_cast<const f32x4*>(&sL[buf][ql]);
          const f32x4 D4 = *reinterpret_cast<const f32x4*>(&sD[buf][ql]);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int r = 4 * i4 + jj;
            float p = exp2_fast(fmaf(s[t][r], c, -L4[jj]));
            if (need_mask) {
              const int q = qb0 + ql + jj;
              if (q >= N || kvrow >= N || (CAUSAL && kvrow > q)) p = 0.f;
            }
            s[t][r] = p;
            dp[t][r] = p * (dp[t][r] - D4[jj]);
          }
        }
      // P^T and dS^T as A operands (lane = key row), K-step st covers queries
      // 16st..16st+15: registers 0..3 <- 16st+4h+jj, 4..7 <- 16st+8+4h+jj
#pragma unroll
      for (int st = 0; st < BR / 16; ++st) {
        const int t = st >> 1, i0 = 2 * (st & 1);
        const bf16x8 pa = pack8(s[t][4 * i0 + 0], s[t][4 * i0 + 1], s[t][4 * i0 + 2], s[t][4 * i0 + 3],
                                s[t][4 * i0 + 4], s[t][4 * i0 + 5], s[t][4 * i0 + 6], s[t][4 * i0 + 7]);
        const bf16x8 da = pack8(dp[t][4 * i0 + 0], dp[t][4 * i0 + 1], dp[t][4 * i0 + 2], dp[t][4 * i0 + 3],
                                dp[t][4 * i0 + 4], dp[t][4 * i0 + 5], dp[t][4 * i0 + 6], dp[t][4 * i0 + 7]);
        const int k0 = 16 * st + 4 * h;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int n0 = 32 * dt + 16 * (g & 1);
          dv[dt] = mfma32(pa, tr_operand<ROWB>(Gt, k0, k0 + 8, n0, lane), dv[dt]);
          dk[dt] = mfma32(da, tr_operand<ROWB>(Qt, k0, k0 + 8, n0, lane), dk[dt]);
        }
      }
      // dS (bf16) to LDS, [key][query]
      const int krow = 32 * wave + l32;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          bf16x4 v;
          v[0] = (bf16)dp[t][4 * i4 + 0];
          v[1] = (bf16)dp[t][4 * i4 + 1];
          v[2] = (bf16)dp[t][4 * i4 + 2];
          v[3] = (bf16)dp[t][4 * i4 + 3];
          *reinterpret_cast<bf16x4*>(&sS[ds_off(krow, 32 * t + 8 * i4 + 4 * h)]) = v;
        }
    } else {
      const int krow = 32 * wave + l32;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          *reinterpret_cast<u32x2*>(&sS[ds_off(krow, 32 * t + 8 * i4 + 4 * h)]) = u32x2{0, 0};
    }
    __syncthreads();
    // dQ_i += dS K over the whole key block: wave takes d-slice dsl and query
    // tiles mt0 .. mt0+NQT-1.  A = dS with the query across lanes (transposing
    // reads of the [key][query] tile), B = K^T slice in registers.
#pragma unroll
    for (int u = 0; u < NQT; ++u) {
      const int mt = mt0 + u;
      if (qb0 + 32 * mt >= N) continue;
      f32x16 acc = f32x16{};
#pragma unroll
      for (int s = 0; s < BC / 16; ++s) {
        const int kr = 16 * s + 8 * h;
        const int scol = lane & 15;
        const int col = 32 * mt + 16 * (g & 1) + 4 * (scol & 3);
        const bf16x4 lo = lds_read_tr(sS, ds_off(kr + (scol >> 2), col));
        const bf16x4 hi = lds_read_tr(sS, ds_off(kr + 4 + (scol >> 2), col));
        acc = mfma32(cat(lo, hi), ktf[s], acc);
      }
      // acc[4*i4+jj] = dQ[query 32mt + 8*i4 + 4h + jj][d 32*dsl + l32]
      float* dst = dQh + (size_t)(qb0 + 32 * mt) * D + 32 * dsl + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = 8 * (r >> 2) + 4 * h + (r & 3);
        if (qb0 + 32 * mt + ql < N) unsafeAtomicAdd(dst + (size_t)ql * D, acc[r]);
      }
    }
    if (i + 1 < nqb) swrite(buf ^ 1);
    __syncthreads();
  }

  // ---- write-back: dK = scale * acc, dV = acc, staged through LDS ----------
  // accumulator r of tile dt: key 32*wave + 8*(r/4) + 4h + r%4, d 32*dt + l32
  bf16* stK = reinterpret_cast<bf16*>(sK);   // [128][D] plain row-major staging
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * wave + 8 * (r >> 2) + 4 * h + (r & 3);
        const float x = pass == 0 ? dk[dt][r] * scale : dv[dt][r];
        stK[row * D + 32 * dt + l32] = (bf16)x;
      }
    __syncthreads();
    bf16* dst = (pass == 0 ? dK : dV) + hoff;
    constexpr int OPT = BC * CH / 256;
#pragma unroll
    for (int p = 0; p < OPT; ++p) {
      const int ci = p * 256 + tid;
      const int row = ci / CH, ch = ci % CH;
      if (kv0 + row < N)
        *reinterpret_cast<u32x4*>(dst + (size_t)(kv0 + row) * D + ch * 8) =
            *reinterpret_cast<const u32x4*>(&stK[row * D + ch * 8]);
    }
    __syncthreads();
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_bwd_bf16_t(const void* q, const void* k, const void* v, const void* dO,
                                    const float* lse2, const float* drow, float* dq_acc, void* dk,
                                    void* dv, int BH, int N, float scale, hipStream_t stream) {
  const int nkb = (N + 127) / 128, nqb = (N + 63) / 64;
  const dim3 grid((unsigned)(nkb * BH)), block(256);
  hipLaunchKernelGGL((bwd_bf16_kernel<D, CAUSAL>), grid, block, 0, stream, (const bf16*)q,
                     (const bf16*)k, (const bf16*)v, (const bf16*)dO, lse2, drow, dq_acc, (bf16*)dk,
                     (bf16*)dv, BH, N, nqb, scale, scale * kLog2e);
  return hipGetLastError();
}

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* dO,
                           const float* lse2, const float* drow, float* dq_acc, void* dk, void* dv,
                           int BH, int N, int d, bool causal, float scale, hipStream_t stream) {
  if (d == 128)
    return causal ? launch_bwd_bf16_t<128, true>(q, k, v, dO, lse2, drow, dq_acc, dk, dv, BH, N, scale, stream)
                  : launch_bwd_bf16_t<128, false>(q, k, v, dO, lse2, drow, dq_acc, dk, dv, BH, N, scale, stream);
  return causal ? launch_bwd_bf16_t<64, true>(q, k, v, dO, lse2, drow, dq_acc, dk, dv, BH, N, scale, stream)
                : launch_bwd_bf16_t<64, false>(q, k, v, dO, lse2, drow, dq_acc, dk, dv, BH, N, scale, stream);
}

}  // namespace fa
