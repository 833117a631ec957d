// fa_bwd_kv2.hip -- the key/value-block-outer backward (dK, dV) at d = 128
// with two waves per SIMD: plain and with the dS stores of the hand-off.
//
// The same method as fa_bwd_kv_body.h (page "flash-attention-backpropagation"
// (aiqz.cc), section QKV梯度; one recompute of P^ per pair of blocks feeding
// all gradients, page "gsyq.cn news/1372000", 踩坑二), with another split of
// the work.  A workgroup of 8 waves owns 128 keys of one (batch, head) and
// walks the query blocks of 64 rows; wave w takes key slice w % 4 (32 keys)
// and query half w / 4 (32 rows) of every block, so that two waves hold the
// same keys and each accumulates dK, dV over its own queries.  Per wave and
// block:
//   S           = Q_h K_w^T - LSE/scale   MFMA, A = Q rows (LDS), B = K rows (LDS)
//   dP          = dO_h V_w^T - D          MFMA, A = dO rows (LDS), B = V rows (LDS)
//   P^ = 2^(c S), dS = P^ o dP            (sections 数值稳定, Softmax梯度)
//   dV_w += P^T dO_h, dK_w += dS^T Q_h    MFMA, A from the S / dP accumulators,
//                                         B through transposing LDS reads
// A wave holds only its dK, dV accumulators (128 registers), one S and one dP
// tile and its operands in flight, at most 256 registers, so two waves share
// each SIMD and the matrix pipe runs one wave's products while the other
// waits for LDS or forms exponentials.  K and V of the block stay in LDS (64
// KB) instead of registers; the Q and dO tiles of a block are fetched straight
// into LDS one block ahead (double buffers), one barrier per block.  At the
// end of a key block the two waves of a slice add their dK, dV through LDS.
// With the hand-off each wave stores its 32 x 32 block of bf16 dS (two 1 KB
// micro-tiles of the DsOut layout) after its products, and the barrier that
// closes the block leaves those stores outstanding.
//
// Not the default (selected with FA_KV_KERNEL=2): on the causal 8192-token,
// 32-head step it runs within about 1% of the one-wave kernel, whose matrix
// pipe it does not keep busier (0.46 against 0.47 of the SIMD cycles).  The
// block barrier aligns the two waves of a SIMD, so both form their
// exponentials at the same time and the pipe idles then, while every operand
// of the products, K and V included, now comes from LDS (1.5 times the LDS
// reads per product).
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

template <bool CAUSAL, bool DSO>
__global__ __launch_bounds__(512, 1) void bwd_kv2_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ NLSE, const float* __restrict__ NDR,
    bf16* __restrict__ dK, bf16* __restrict__ dV, int BH, int N, int nqb, float scale, float c, Layouts lay,
    DsOut dso) {
  constexpr int D = 128, BC = 128, BR = 64;
  constexpr int ROWB = lds_pitch<D>(), KS = D / 16, DT = D / 32;
  constexpr int QTB = BR * ROWB, KTB = BC * ROWB;

  // One LDS array at fixed offsets: the query tiles (read with per-lane bases
  // that include the wave's query half) in the first 64 KB, the key block
  // after them, so that every operand read is one of a few per-lane bases plus
  // an offset that fits the 16-bit immediate of a ds_read.
  constexpr int OQ0 = 0, OQ1 = QTB, OG0 = 2 * QTB, OG1 = 3 * QTB;   // Q, dO tiles (two buffers each)
  constexpr int OK = 4 * QTB, OV = OK + KTB;                        // K, V of the key block
  constexpr int OL = OV + KTB;                                      // -LSE/scale, -D rows (two buffers each)
  static_assert(OK == 65536, "query tiles fill the first 64 KB");
  __shared__ __attribute__((aligned(1024))) char lds[OL + 4 * BR * 4];
  char* const sQ0 = lds + OQ0;
  char* const sQ1 = lds + OQ1;
  char* const sG0 = lds + OG0;   // dO
  char* const sG1 = lds + OG1;
  char* const sK = lds + OK;
  char* const sV = lds + OV;
  float* const sL0 = reinterpret_cast<float*>(lds + OL);            // -LSE / scale
  float* const sL1 = sL0 + BR;
  float* const sD0 = sL0 + 2 * BR;                                  // -D
  float* const sD1 = sL0 + 3 * BR;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slice = wave_u & 3, qh = wave_u >> 2;   // key slice, query half
  const TileFetch<ROWB, BR, 8> qfetch(wave_u, lane, lay.q.sn * 2);    // Q rows; dO rows at grs
  const unsigned grs = (unsigned)lay.g.sn * 2u, vrs = (unsigned)lay.v.sn * 2u;
  // work items as in fa_bwd_kv_body.h: causal item c is the key-block pair
  // (c, nkb-1-c), the first walked downward, the second upward; XCD-major
  // numbering keeps the items of a head on one XCD's L2
  const int nkb = (N + BC - 1) / BC;
  const int P = CAUSAL ? (nkb + 1) / 2 : nkb;
  const int W = P * BH;
  const int bid = blockIdx.x;
  const int item = (W % 8 == 0) ? (bid % 8) * (W / 8) + bid / 8 : bid;
  const int head = item / P, c_item = item % P;
  const int nparts = (CAUSAL && 2 * c_item + 1 != nkb) ? 2 : 1;
  const bf16* Qh = Q + lay.off(lay.q, head);
  const bf16* Kh = K + lay.off(lay.k, head);
  const bf16* Vh = V + lay.off(lay.v, head);
  const bf16* Gh = dO + lay.off(lay.g, head);
  const float* Lh = NLSE + (size_t)head * N;
  const float* Dh = NDR + (size_t)head * N;

  auto run_part = [&](int part) {
    int ln = lane;
    asm volatile("" : "+v"(ln));   // lane-dependent addresses re-derived per part
    const int l32 = ln & 31, h = ln >> 5;
    const int kb = CAUSAL ? (part == 0 ? c_item : nkb - 1 - c_item) : c_item;
    const bool ascend = part == 1;
    const int kv0 = kb * BC;
    const int kvw = kv0 + 32 * slice;   // first key of this wave
    const int kvrow = kvw + l32;        // key of this lane in the S accumulators

    char* dsw = nullptr;
    if constexpr (DSO) dsw = dso.buf + (size_t)head * dso.head_bytes + (size_t)(kv0 / 32 + slice) * 4096u;

    // per-lane bases: natural operands (lane = row 32*qh + l32 of a query
    // tile; chunk 2ks + h) and the transposed reads of the query tiles (rows
    // 32*qh + 16*hi + ..., column group dt), each plus a compile-time offset.
    // The key block's rows 32*slice + l32 sit a per-wave distance after the
    // query rows of the same ks, added per K-step (eight more live address
    // registers would not fit).
    int rq[KS], rt[DT][2];
    {
      const TileBases<ROWB> tb(ln);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) rq[ks] = tb.nat_off(0, ks) + 32 * ROWB * qh;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int hi = 0; hi < 2; ++hi) rt[dt][hi] = tb.tr_off(0, dt, hi) + 32 * ROWB * qh;
    }
    const int i_begin = CAUSAL ? (kv0 / BR) : 0;
    auto fetch = [&](int i, char* dQt, char* dGt, float* dL, float* dD) {
      const int qb0 = i * BR;
      qfetch(Qh, qb0, N, dQt);
      qfetch(Gh, qb0, N, dGt, grs);
      if (qb0 + BR <= N) {
        if (wave_u == 0) dma4_buf(raw_rsrc(Lh), 4 * ln, 4 * qb0, dL);
        if (wave_u == 1) dma4_buf(raw_rsrc(Dh), 4 * ln, 4 * qb0, dD);
      } else {
        if (wave_u == 0) dma4_buf(raw_rsrc(Lh), 4 * min(qb0 + ln, N - 1), 0, dL);
        if (wave_u == 1) dma4_buf(raw_rsrc(Dh), 4 * min(qb0 + ln, N - 1), 0, dD);
      }
    };

    f32x16 dk[DT], dv[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      dk[t] = f32x16{};
      dv[t] = f32x16{};
    }

    const int nsteps = nqb - i_begin;
    auto body = [&](auto bc, int k) {
      constexpr int b = decltype(bc)::value;
      const int i = ascend ? i_begin + k : nqb - 1 - k;
      constexpr int OQ = b ? OQ1 : OQ0, OG = b ? OG1 : OG0;
      const float* Lt = b ? sL1 : sL0;
      const float* Dt = b ? sD1 : sD0;
      const int dir = ascend ? 1 : -1;
      if (k + 1 < nsteps) fetch(i + dir, b ? sQ0 : sQ1, b ? sG0 : sG1, b ? sL0 : sL1, b ? sD0 : sD1);
      FA_DEBUG_BARRIER();
      __builtin_amdgcn_sched_barrier(0);
      const int qb0 = i * BR, q0 = qb0 + 32 * qh;   // this wave's first query
      // the wave's keys all come after its queries: P^ = 0, nothing to add
      const bool dead = (kvw >= N) || (q0 >= N) || (CAUSAL && q0 + 31 < kvw);
      // the hand-off stores the dS of every 32-key slice that reaches the
      // diagonal of the 64-row block (the buffer's layout), zeros where masked;
      // a slice wholly after the block goes to the sink.  Every wave issues the
      // same two stores, a dead wave's being zeros.
      const bool to_sink = (kvw >= N) || (CAUSAL && qb0 + BR - 1 < kvw);
      bf16x8 da_keep[2];
      // the mask is applied in place behind a uniform branch: a second copy
      // of the block's code for masked blocks pushes the wave past 256
      // registers
      const bool need_mask = (CAUSAL && q0 < kvw + 31) || (q0 + 32 > N) || (kvw + 32 > N);
      auto compute = [&] {
        // accumulators start from -LSE/scale and -D of the query rows:
        // register r is query q0 + 8*(r/4) + 4h + r%4
        f32x16 s, dp;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int ql = 32 * qh + 8 * i4 + 4 * h;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(Lt + ql);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(Dt + ql);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            s[4 * i4 + jj] = l4[jj];
            dp[4 * i4 + jj] = d4[jj];
          }
        }
        // S = Q_h K_w^T, dP = dO_h V_w^T over the 8 K-steps of d, the
        // operands read one K-step ahead.  Scheduling fences around each
        // step's reads keep them ahead of its products and stop the compiler
        // from hoisting all of them (128 registers); the other wave on the
        // SIMD covers what remains of the read latency.  kd passes through an
        // empty asm inside the block so that the key addresses are formed per
        // K-step instead of being hoisted out of the walk.
        bf16x8 op[4];
        int kd = OK + 32 * ROWB * (slice - qh);
        asm volatile("" : "+s"(kd));
        auto rd = [&](int ks) {
          const int rk = rq[ks] + kd;
          op[0] = lds_read_b128(lds + OQ, rq[ks]);
          op[1] = lds_read_b128(lds, rk);
          op[2] = lds_read_b128(lds + OG, rq[ks]);
          op[3] = lds_read_b128(lds + KTB, rk);
        };
        rd(0);
        // raised issue priority while the wave runs its products, so that a
        // wave in its product phase wins the arbitration against the other
        // wave's exponentials (measured: about 3% on the causal 8192-token
        // step against no priority change)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          __builtin_amdgcn_sched_barrier(0);
          const bf16x8 a0 = op[0], b0 = op[1], a1 = op[2], b1 = op[3];
          if (ks + 1 < KS) rd(ks + 1);
          __builtin_amdgcn_sched_barrier(0);
          s = mfma32(a0, b0, s);
          dp = mfma32(a1, b1, dp);
          asm volatile("" : "+v"(s), "+v"(dp));
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        // P^ and dS; operands of dV, dK: K-step hi covers queries
        // 16hi..16hi+15 of the wave's 32
        bf16x8 pa[2], da[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = exp2_fast(s[r] * c);
        if (need_mask) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int q = q0 + 8 * (r >> 2) + 4 * h + (r & 3);
            const bool masked = (q >= N) | (kvrow >= N) | (CAUSAL & (kvrow > q));
            s[r] = masked ? 0.f : s[r];
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[r] = s[r] * dp[r];
#pragma unroll
        for (int hi = 0; hi < 2; ++hi) {
          const int o = 8 * hi;
          pa[hi] = pack8(s[o], s[o + 1], s[o + 2], s[o + 3], s[o + 4], s[o + 5], s[o + 6], s[o + 7]);
          da[hi] = pack8(dp[o], dp[o + 1], dp[o + 2], dp[o + 3], dp[o + 4], dp[o + 5], dp[o + 6], dp[o + 7]);
        }
        // dV += P^T dO_h, dK += dS^T Q_h, the transposed operands read one
        // product pair ahead
        bf16x8 tp[2];
        auto rdt = [&](int j) {
          const int hi = j / DT, dt = j % DT;
          const int o0 = rt[dt][0] + 16 * ROWB * hi, o1 = rt[dt][1] + 16 * ROWB * hi;
          tp[0] = cat(lds_read_tr(lds + OG, o0), lds_read_tr(lds + OG, o1));
          tp[1] = cat(lds_read_tr(lds + OQ, o0), lds_read_tr(lds + OQ, o1));
        };
        rdt(0);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int j = 0; j < 2 * DT; ++j) {
          __builtin_amdgcn_sched_barrier(0);
          const int hi = j / DT, dt = j % DT;
          const bf16x8 tg = tp[0], tq = tp[1];
          if (j + 1 < 2 * DT) rdt(j + 1);
          __builtin_amdgcn_sched_barrier(0);
          dv[dt] = mfma32(pa[hi], tg, dv[dt]);
          dk[dt] = mfma32(da[hi], tq, dk[dt]);
          asm volatile("" : "+v"(dv[dt]), "+v"(dk[dt]));
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        if constexpr (DSO) {
          da_keep[0] = da[0];
          da_keep[1] = da[1];
        }
      };
      if (!dead) {
        compute();
      } else if constexpr (DSO) {
        da_keep[0] = bf16x8{};
        da_keep[1] = bf16x8{};
      }
      if constexpr (DSO) {
        char* p = (to_sink ? dso.sink : dsw + ds_block_off(CAUSAL, i, dso.nks)) + 16 * ln + 1024 * (2 * qh);
        __builtin_nontemporal_store(da_keep[0], reinterpret_cast<bf16x8*>(p));
        __builtin_nontemporal_store(da_keep[1], reinterpret_cast<bf16x8*>(p + 1024));
        // s_waitcnt vmcnt(2) lgkmcnt(0): all but the two stores; no fence (a
        // release fence would wait for them too)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0x0072);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      } else {
        __syncthreads();
      }
    };

    // the key block into LDS, then the first query block
    {
      const TileFetch<ROWB, BC, 8> kfetch(wave_u, ln, lay.k.sn * 2);   // K rows; V rows at vrs
      kfetch(Kh, kv0, N, sK);
      kfetch(Vh, kv0, N, sV, vrs);
    }
    if (nsteps > 0) fetch(ascend ? i_begin : nqb - 1, sQ0, sG0, sL0, sD0);
    __syncthreads();
    if (nsteps > 0) {
      int k = 0;
      while (true) {
        body(IC<0>{}, k);
        if (++k >= nsteps) break;
        body(IC<1>{}, k);
        if (++k >= nsteps) break;
      }
    }

    // ---- the two query halves' dK, dV summed, then written ---------------------
    // fp32 partials of half the columns at a time through sK (idle after the
    // walk), laid out [slice][register][lane] so that each lane moves 4-byte
    // words without bank conflicts: qh = 1 hands its dK to qh = 0, and qh = 0
    // its dV to qh = 1.  Each wave then stages its 32 rows as bf16 ([32][128]
    // row-major, 8 KB: qh = 0 in sK, qh = 1 in sV) for 16-byte row stores.
    float* red = reinterpret_cast<float*>(sK) + slice * (32 * 64);   // 8 KB per slice
    auto exchange = [&](f32x16 (&mine)[DT], bool give) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        if (give) {
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e) red[(16 * t + e) * 64 + ln] = mine[2 * half + t][e];
        }
        __syncthreads();
        if (!give) {
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e) mine[2 * half + t][e] += red[(16 * t + e) * 64 + ln];
        }
        __syncthreads();
      }
    };
    exchange(dk, qh == 1);   // qh = 0 holds the sum of dK
    exchange(dv, qh == 0);   // qh = 1 holds the sum of dV
    auto write_rows = [&](const f32x16 (&acc)[DT], float mul, char* region, bf16* dst, int ors) {
      bf16* stg = reinterpret_cast<bf16*>(region);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 8 * (r >> 2) + 4 * h + (r & 3);
          stg[row * D + 32 * dt + l32] = (bf16)(acc[dt][r] * mul);
        }
      constexpr int CW = D / 8, OPW = 32 * CW / 64;   // 16-byte chunks per row, stores per lane
#pragma unroll
      for (int p = 0; p < OPW; ++p) {
        const int ci = p * 64 + ln;
        const int row = ci / CW, ch = ci % CW;
        if (kvw + row < N)
          *reinterpret_cast<u32x4*>(dst + (size_t)(kvw + row) * ors + ch * 8) =
              *reinterpret_cast<const u32x4*>(&stg[row * D + ch * 8]);
      }
    };
    if (qh == 0)
      write_rows(dk, scale, sK + slice * (32 * ROWB), dK + lay.off(lay.dk, head), lay.dk.sn);
    else
      write_rows(dv, 1.f, sV + slice * (32 * ROWB), dV + lay.off(lay.dv, head), lay.dv.sn);
    __syncthreads();   // the next part refills every buffer
  };
  run_part(0);
  if (nparts > 1) run_part(1);
}

hipError_t launch_bwd_kv2(const void* q, const void* k, const void* v, const void* dO, const float* nlse,
                          const float* ndrow, void* dk, void* dv, int BH, int N, bool causal, float scale,
                          Layouts lay, hipStream_t stream, DsOut ds) {
  constexpr int BC = 128;
  const int nkb = (N + BC - 1) / BC, nqb = (N + 63) / 64;
  const int items = causal ? (nkb + 1) / 2 : nkb;
  const dim3 grid((unsigned)(items * BH)), block(512);
  const float c = ledger_scale(scale) * kLog2e;   // dK keeps the caller's scale
  auto go = [&](auto kern, DsOut d) {
    hipLaunchKernelGGL(kern, grid, block, 0, stream, (const bf16*)q, (const bf16*)k, (const bf16*)v,
                       (const bf16*)dO, nlse, ndrow, (bf16*)dk, (bf16*)dv, BH, N, nqb, scale, c, lay, d);
  };
  if (ds.buf) {
    if (causal) go(bwd_kv2_kernel<true, true>, ds);
    else go(bwd_kv2_kernel<false, true>, ds);
  } else {
    if (causal) go(bwd_kv2_kernel<true, false>, DsOut{});
    else go(bwd_kv2_kernel<false, false>, DsOut{});
  }
  return hipGetLastError();
}

}  // namespace fa
