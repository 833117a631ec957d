// fa_bwd_dq.hip -- query-block-outer dQ kernel, bf16 in/out, fp32 accumulation.
//
// dQ_i = scale * sum_j dS_ij K_j (page "flash-attention-backpropagation"
// (aiqz.cc), section QKV梯度), computed without atomics: one workgroup
// (8 waves, two per SIMD; d = 256: 4 waves, one per SIMD) owns BR = 256 (128)
// query rows of one (batch, head), each wave 32 of them, with the wave's Q and dO rows in registers and dQ accumulated in
// registers, and walks the key/value tiles of BC = 64 rows (double-buffered
// through LDS).  Per tile and wave:
//   S^T  = K_j Q_w^T           MFMA, A = K rows (LDS), B = Q_w (registers)
//   dP^T = V_j dO_w^T          MFMA, A = V rows (LDS), B = dO_w (registers)
//   P^   = 2^(c*(S - LSE/scale))  recompute from the ledger (section 数值稳定);
//                              the lane holds one query row, so LSE and D
//                              are per-lane scalars
//   dS   = P^ o (dP - D)       (section Softmax梯度); the dP accumulator
//                              starts from -D
//   dQ^T += K_j^T dS^T         MFMA, A = K^T through transposing LDS reads,
//                              B = dS^T straight from the accumulators.
// It repeats the S and dP products of the key/value-outer kernel instead of
// exchanging dS through fp32 atomics.  Each 32-key half of a tile is a fixed
// sequence of slots separated by scheduling fences, with the LDS operands of
// each slot read a few slots ahead.
#include "fa_common.h"
#include "fa_dropout.h"
#include "fa_launch.h"

namespace fa {

#ifndef FA_DQ_NW
#define FA_DQ_NW 8
#endif
// The kernel body, shared by the plain kernel and the dropout kernel (DROP:
// with keep mask Z and keep scale s, dP = s Z o (dO V^T), so that
// dS = P^ o (s (dP~ - D) + (s - 1) D) where kept and P^ o (-D) where dropped,
// dP~ - D being what the dP accumulator holds).
template <int D, bool CAUSAL, int NW, bool DROP>
FA_DEV void bwd_dq_body(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
                        const bf16* __restrict__ dO, const float* __restrict__ NLSE,
                        const float* __restrict__ NDR, bf16* __restrict__ dQ, int BH, int N, int nqb,
                        float scale, float c, Layouts lay, DropArgs dr) {
  constexpr int BR = 32 * NW, BC = 64;
  constexpr int ROWB = lds_pitch<D>();   // LDS bytes per row (d * 2, or 256 for d = 96)
  constexpr int KS = D / 16;         // K-steps of the S and dP products
  constexpr int DT = D / 32;         // 32-row tiles of dQ^T
  constexpr int TILEB = BC * ROWB;   // bytes of one K or V tile

  __shared__ __attribute__((aligned(1024))) char sK0[TILEB];
  __shared__ __attribute__((aligned(1024))) char sK1[TILEB];
  __shared__ __attribute__((aligned(1024))) char sV0[TILEB];
  __shared__ __attribute__((aligned(1024))) char sV1[TILEB];

  // the wave index is uniform across the wave; readfirstlane tells the compiler
  // so, which keeps the wave-level conditions below scalar branches
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5;
  const TileBases<ROWB> tb(lane);
  const TileFetch<ROWB, BC, NW, D / 8> fetch(wave, lane, lay.k.sn * 2);   // K rows; V rows at vrs
  const unsigned vrs = (unsigned)lay.v.sn * 2u;
  const int bid = blockIdx.x;
  const int head = bid % BH;
  // causal: the longest query blocks are dispatched first
  const int qb = CAUSAL ? (nqb - 1 - bid / BH) : (bid / BH);
  const bf16* Qh = Q + lay.off(lay.q, head);
  const bf16* Kh = K + lay.off(lay.k, head);
  const bf16* Vh = V + lay.off(lay.v, head);
  const bf16* Gh = dO + lay.off(lay.g, head);

  const int q0 = qb * BR + wave * 32;   // first query row of this wave
  const int qrow = q0 + l32;            // the query row this lane's statistics belong to

  // Q and dO rows as B operands: lane (n = l32, half h) holds d = 16*s + 8*h + r
  bf16x8 qf[KS], gf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (qrow < N) {
      qf[s] = *reinterpret_cast<const bf16x8*>(Qh + (size_t)qrow * lay.q.sn + 16 * s + 8 * h);
      gf[s] = *reinterpret_cast<const bf16x8*>(Gh + (size_t)qrow * lay.g.sn + 16 * s + 8 * h);
    } else {
      qf[s] = bf16x8{};
      gf[s] = bf16x8{};
    }
  }
  // -LSE * log2(e) and -D of this lane's query row
  const float nl2 = qrow < N ? NLSE[(size_t)head * N + qrow] * c : 0.f;
  const float ndrow = qrow < N ? NDR[(size_t)head * N + qrow] : 0.f;
  // dropout: a kept dS is P^ (s acc + (1 - s) ndrow), with acc = dP~ + ndrow
  const float kd = DROP ? (1.f - dr.keep_scale) * ndrow : 0.f;

  const int kv_end = CAUSAL ? min(N, qb * BR + BR) : N;
  const int ntiles = (kv_end + BC - 1) / BC;
  int wave_tiles = 0;
  if (q0 < N) {
    const int wkv_end = CAUSAL ? min(N, q0 + 32) : N;
    wave_tiles = (wkv_end + BC - 1) / BC;
  }


  f32x16 acc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) acc[t] = f32x16{};

  // one key/value tile: products from buffer b while tile j+1 is fetched
  // straight into buffer b^1 (distinct LDS objects per buffer, so the fetch
  // cannot alias the reads)
  auto body = [&](auto bc, int j) {
    constexpr int b = decltype(bc)::value;
    const char* Kt = b ? sK1 : sK0;
    const char* Vt = b ? sV1 : sV0;
    if (j + 1 < ntiles) {
      fetch(Kh, (j + 1) * BC, N, b ? sK0 : sK1);
      fetch(Vh, (j + 1) * BC, N, b ? sV0 : sV1, vrs);
      FA_DEBUG_BARRIER();
    }
    if (j < wave_tiles) {
      const int kvb = j * BC;
      const bool need_mask = (kvb + BC > N) || (CAUSAL && kvb + BC - 1 > q0) || (q0 + 32 > N);
      // The tile's two 32-key halves one after the other (fewer live
      // registers), each as: S, dP products (KS slots of two products), the
      // exponentials, the dQ products (2*DT slots of one product).  Slot i
      // issues the LDS reads of slot i + DIST before its products, with
      // scheduling fences between slots, so each product waits only for reads
      // issued DIST slots earlier (LDS returns in order).
#ifndef FA_DQ_DIST
#define FA_DQ_DIST 3
#endif
      constexpr int DIST = FA_DQ_DIST;   // slots between an LDS read and its use
      constexpr int SPM = KS + 2 * DT;    // slots per 32-key half
      constexpr int NSL = 2 * SPM;
      bf16x8 ka[KS], va[KS], kt[2 * DT];
      auto read_slot = [&](int i) {
        const int mt = i / SPM, k = i % SPM;
        if (k < KS) {
          const int off = tb.nat_off(mt, k);
          ka[k] = lds_read_b128(Kt, off);
          va[k] = lds_read_b128(Vt, off);
        } else {
          const int u = k - KS, half = u / DT, t = u % DT;
          const int st = 2 * mt + half;
          kt[u] = cat(lds_read_tr(Kt, tb.tr_off(st, t, 0)), lds_read_tr(Kt, tb.tr_off(st, t, 1)));
        }
      };
      f32x16 s, dp;
      bf16x8 db[2];
      // dropout: the generator of this lane quad's 4x4 block in key group
      // lane % 4 of the current 32-key half; its rounds run in the half's
      // S/dP slots
      Philox4 ph;
#pragma unroll
      for (int i = 0; i < DIST; ++i) read_slot(i);
      // full unrolling is required (every register array index below is a
      // compile-time constant); at d = 256 the body is past the size up to
      // which a plain unroll pragma is honoured
#pragma clang loop unroll(full)
      for (int i = 0; i < NSL; ++i) {
        const int mt = i / SPM, k = i % SPM;
        __builtin_amdgcn_sched_barrier(0);
        if (i + DIST < NSL) read_slot(i + DIST);
        if (k < KS) {
          if (k == 0) {
            if constexpr (DROP)
              ph = Philox4{(uint32_t)(kvb + 32 * mt + 8 * (lane & 3) + 4 * h) >> 2, (uint32_t)qrow >> 2,
                           (uint32_t)head, dr.offset};
            s = f32x16{};
            // dP starts from -D of this lane's query row, so that the products
            // leave dP - D (every register of the lane belongs to that row)
#pragma unroll
            for (int r = 0; r < 16; ++r) dp[r] = ndrow;
          }
          s = mfma32(ka[k], qf[k], s);
          dp = mfma32(va[k], gf[k], dp);
          if constexpr (DROP) ph.rounds(10 * k / KS, 10 * (k + 1) / KS, dr.k0, dr.k1);
          if (k == KS - 1) {
            __builtin_amdgcn_sched_barrier(0);
            // register r: key kvb + 32*mt + 8*(r/4) + 4*h + r%4, query qrow.
            // Masked scores become an infinity of c's opposite sign (c s = -inf,
            // P^ = 0; c < 0 for a negative scale), behind one uniform branch.
            if (need_mask) {
              const float dead_s = c > 0.f ? -INFINITY : INFINITY;
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int kv = kvb + 32 * mt + 8 * (r >> 2) + 4 * h + (r & 3);
                const bool dead = (kv >= N) | (qrow >= N) | (CAUSAL & (kv > qrow));
                s[r] = dead ? dead_s : s[r];
              }
            }
            if constexpr (DROP) {
              const u32x4 w = quad_transpose(ph.words(), lane & 3);
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const float p = exp2_fast(fmaf(s[r], c, nl2));
                dp[r] = p * (kept(w[r >> 2], r & 3, dr.thresh) ? fmaf(dr.keep_scale, dp[r], kd) : ndrow);
              }
            } else {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const float p = exp2_fast(fmaf(s[r], c, nl2));
                dp[r] = p * dp[r];
              }
            }
            // dS^T as B operand; K-step st = 2*mt + half covers keys 16*st ..
            // 16*st+15 of the tile: registers 0..3 <- keys 16st+4h+jj, 4..7 <-
            // keys 16st+8+4h+jj
#pragma unroll
            for (int half = 0; half < 2; ++half) {
              const int i0 = 2 * half;
              db[half] = pack8(dp[4 * i0 + 0], dp[4 * i0 + 1], dp[4 * i0 + 2], dp[4 * i0 + 3],
                               dp[4 * i0 + 4], dp[4 * i0 + 5], dp[4 * i0 + 6], dp[4 * i0 + 7]);
            }
          }
        } else {
          const int u = k - KS, half = u / DT, t = u % DT;
          acc[t] = mfma32(kt[u], db[half], acc[t]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
  };

  fetch(Kh, 0, N, sK0);
  fetch(Vh, 0, N, sV0, vrs);
  __syncthreads();
  for (int j = 0;;) {
    body(IC<0>{}, j);
    if (++j >= ntiles) break;
    body(IC<1>{}, j);
    if (++j >= ntiles) break;
  }

  if (qrow >= N) return;
  // acc[t][4*i+jj] = dQ^T[d = 32t + 8i + 4h + jj][query qrow]
  bf16* row = dQ + lay.off(lay.dq, head) + (size_t)qrow * lay.dq.sn;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x4 v;
      v[0] = (bf16)(acc[t][4 * i + 0] * scale);
      v[1] = (bf16)(acc[t][4 * i + 1] * scale);
      v[2] = (bf16)(acc[t][4 * i + 2] * scale);
      v[3] = (bf16)(acc[t][4 * i + 3] * scale);
      *reinterpret_cast<bf16x4*>(row + 32 * t + 8 * i + 4 * h) = v;
    }
}

// waves per SIMD the kernel is built for: at d = 256 the wave's Q and dO rows
// and its dQ accumulator alone take 256 registers
template <int D, int NW>
constexpr int dq_min_blocks() {
  return D > 128 ? 4 / NW : 8 / NW;
}

template <int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(64 * NW, (dq_min_blocks<D, NW>())) void bwd_dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ NLSE, const float* __restrict__ NDR,
    bf16* __restrict__ dQ, int BH, int N, int nqb, float scale, float c, Layouts lay) {
  bwd_dq_body<D, CAUSAL, NW, false>(Q, K, V, dO, NLSE, NDR, dQ, BH, N, nqb, scale, c, lay, DropArgs{});
}

template <int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(64 * NW, (dq_min_blocks<D, NW>())) void bwd_dq_dropout_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ NLSE, const float* __restrict__ NDR,
    bf16* __restrict__ dQ, int BH, int N, int nqb, float scale, float c, Layouts lay, DropArgs dr) {
  bwd_dq_body<D, CAUSAL, NW, true>(Q, K, V, dO, NLSE, NDR, dQ, BH, N, nqb, scale, c, lay, dr);
}

template <int D, bool CAUSAL>
static hipError_t launch_bwd_dq_t(const void* q, const void* k, const void* v, const void* dO,
                                  const float* nlse, const float* ndrow, void* dq, int BH, int N, float scale,
                                  Layouts lay, hipStream_t stream, const DropArgs* drop) {
  constexpr int NW = D == 256 ? 4 : FA_DQ_NW, BR = 32 * NW;   // d = 256: one wave per SIMD
  const int nqb = (N + BR - 1) / BR;
  const dim3 grid((unsigned)(nqb * BH)), block(64 * NW);
  const float c = ledger_scale(scale) * kLog2e;   // dQ keeps the caller's scale
  if (drop) {
    hipLaunchKernelGGL((bwd_dq_dropout_kernel<D, CAUSAL, NW>), grid, block, 0, stream, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, (const bf16*)dO, nlse, ndrow, (bf16*)dq, BH, N, nqb,
                       scale, c, lay, *drop);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, NW>), grid, block, 0, stream, (const bf16*)q, (const bf16*)k,
                     (const bf16*)v, (const bf16*)dO, nlse, ndrow, (bf16*)dq, BH, N, nqb, scale, c, lay);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* dO, const float* nlse,
                         const float* ndrow, void* dq, int BH, int N, int d, bool causal, float scale,
                         Layouts lay, hipStream_t stream, const DropArgs* drop) {
  if (d == 128)
    return causal ? launch_bwd_dq_t<128, true>(q, k, v, dO, nlse, ndrow, dq, BH, N, scale, lay, stream, drop)
                  : launch_bwd_dq_t<128, false>(q, k, v, dO, nlse, ndrow, dq, BH, N, scale, lay, stream, drop);
  if (d == 256)
    return causal ? launch_bwd_dq_t<256, true>(q, k, v, dO, nlse, ndrow, dq, BH, N, scale, lay, stream, drop)
                  : launch_bwd_dq_t<256, false>(q, k, v, dO, nlse, ndrow, dq, BH, N, scale, lay, stream, drop);
  if (d == 96)
    return causal ? launch_bwd_dq_t<96, true>(q, k, v, dO, nlse, ndrow, dq, BH, N, scale, lay, stream, drop)
                  : launch_bwd_dq_t<96, false>(q, k, v, dO, nlse, ndrow, dq, BH, N, scale, lay, stream, drop);
  return causal ? launch_bwd_dq_t<64, true>(q, k, v, dO, nlse, ndrow, dq, BH, N, scale, lay, stream, drop)
                : launch_bwd_dq_t<64, false>(q, k, v, dO, nlse, ndrow, dq, BH, N, scale, lay, stream, drop);
}

}  // namespace fa
