// fa_bwd_kv_body.h -- the key/value-block-outer backward kernel (dK, dV), bf16
// inputs/outputs, fp32 accumulation, d = 64, 96 and 128; instantiated by
// fa_bwd_bf16.hip (d = 256 has a kernel of its own, fa_bwd_kv256_body.h).
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
//   P^ = 2^(c*(S - LSE/scale))     recompute from the ledger (section 数值稳定)
//   dS = P^ o (dP - D)             (section Softmax梯度)
//   dV_w += P^T dO_i               MFMA, A = P^T from the S accumulators,
//                                  B = dO through transposing LDS reads
//   dK_w += dS^T Q_i               MFMA, same shape with dS and Q
//   dQ_i += dS K                   only in the atomic-dQ variant: dS goes
//                                  through LDS (it is needed with the query
//                                  index across lanes); each wave takes a
//                                  32-column slice of d with K^T held in
//                                  registers; fp32 atomics into an accumulator.
// In the hand-off variant (DSO) the bf16 dS operands of every block are also
// stored to a buffer (layout: DsOut in fa_launch.h), from which a separate
// kernel forms dQ = dS K without recomputing S and dP:
//  - the four 16-byte stores of a step follow the step's products, after the
//    masked and unmasked paths join (stores inside the two paths leave the
//    compiler counting 0, 4 or 8 of them; holding dS into the next step made
//    its register use jump past the file);
//  - the barrier closing the step does not wait for them: vector memory
//    operations retire in issue order, so once at most those stores are
//    outstanding the prefetch issued before them has landed in LDS, and the
//    barrier waits for that and for the wave's LDS reads only (a workgroup
//    barrier with a full fence would wait for the stores too);
//  - a wave whose keys all lie past the block's queries runs the masked step
//    anyway (dS = 0; the waves of a workgroup move in step, so it costs no
//    time) and stores to a sink, so that every path issues the same stores;
//  - the stores are non-temporal: nothing here reads them back (measured: the
//    dQ kernel then reads the buffer 7% faster, this kernel is unchanged).
// The S and dP accumulators start from -LSE/scale and -D of their query rows,
// so they end as S - LSE/scale and dP - D.
// The accumulators hold fp32 and are converted once at write-back (page
// "gsyq.cn news/1372000", 踩坑三).  scale is applied to dK here and to dQ by
// the conversion kernel.
//
// Pipelining: Q/dO/LSE/D of the next query block are fetched straight into
// the other LDS buffer (buffer loads into LDS) while the current block is
// used; one barrier per block.  Within a block the work is a fixed sequence of
// 32 slots separated by scheduling fences (products, the LDS reads of the slot
// three ahead, a share of the exponentials).  In the atomic-dQ variant the dQ
// product of a block runs at the start of the next iteration so that its
// atomics drain under the next block's products.  The loop body is
// instantiated per buffer so that every LDS buffer is a distinct object (the
// compiler then knows the prefetch cannot alias the reads).  LDS addresses are
// a few per-lane bases plus compile-time offsets.
#pragma once
#include "fa_common.h"
#include "fa_dropout.h"
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

// The kernel body, shared by the plain kernels and the dropout kernel (DROP:
// with keep mask Z and keep scale s, dV = s (P^ o Z)^T dO and
// dS = P^ o (s (dP~ - D) + (s - 1) D) where kept, P^ o (-D) where dropped,
// dP~ - D being what the dP accumulator holds).
template <int D, bool CAUSAL, bool DQA, bool DROP, bool DSO>
FA_DEV void bwd_bf16_body(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
                          const bf16* __restrict__ dO, const float* __restrict__ NLSE,
                          const float* __restrict__ NDR, float* __restrict__ dQacc, bf16* __restrict__ dK,
                          bf16* __restrict__ dV, int BH, int N, int nqb, float scale, float c, Layouts lay,
                          DropArgs dr, DsOut dso) {
  static_assert(!(DQA && DROP), "the dropout backward takes dQ from another kernel");
  static_assert(!(DQA && DSO), "dQ comes from atomics or from the hand-off, not both");
  static_assert(D == 64 || D == 96 || D == 128, "head dims of this kernel");
  // each wave owns a 32-key slice; a workgroup of 4 waves owns BC keys
  constexpr int BC = 128, BR = 64;
  // ROWB: LDS bytes per row (d * 2, or 256 for d = 96); CH: 16-byte chunks per row
  constexpr int ROWB = lds_pitch<D>(), CH = D / 8, KS = D / 16, DT = D / 32;
  constexpr int DTW = DT;   // 32-column tiles of dK, dV per wave
  static_assert(!DQA || (D == 64 || D == 128), "the atomic dQ variant splits d into 32-column slices over 4 waves");
  constexpr int QTB = BR * ROWB;          // bytes of one Q or dO tile
  constexpr int NQT = (D == 128) ? 2 : 1; // query tiles of dQ per wave

  __shared__ __attribute__((aligned(1024))) char sQ0[QTB];
  __shared__ __attribute__((aligned(1024))) char sQ1[QTB];
  __shared__ __attribute__((aligned(1024))) char sG0[QTB];   // dO
  __shared__ __attribute__((aligned(1024))) char sG1[QTB];
  __shared__ __attribute__((aligned(256))) float sL0[BR];    // -LSE / scale
  __shared__ __attribute__((aligned(256))) float sL1[BR];
  __shared__ __attribute__((aligned(256))) float sD0[BR];    // -D
  __shared__ __attribute__((aligned(256))) float sD1[BR];
  constexpr int SSB = DQA ? BC * BR * 2 : 16;   // dS tiles exist only with atomic dQ
  constexpr int SKB = DQA ? BC * ROWB : 16;      // K block for the K^T operand of dQ
  __shared__ __attribute__((aligned(1024))) char sS0[SSB];  // dS, [key][query]
  __shared__ __attribute__((aligned(1024))) char sS1[SSB];
  __shared__ __attribute__((aligned(1024))) char sK[SKB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slice = wave;   // 32-key slice
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);   // the same value, known uniform
  const TileFetch<ROWB, BR, 4, CH> qfetch(wave_u, lane, lay.q.sn * 2);   // Q rows; dO rows at grs
  const unsigned grs = (unsigned)lay.g.sn * 2u;
  // Work items.  Causal: item c of a head is the key-block pair
  // (c, nkb-1-c), whose query walks together always cover the same number of
  // blocks, so every workgroup does the same work; the first block is walked
  // from the last query block down, the second from its first query block
  // up, so at any moment the workgroups of a head sit on only two query
  // blocks (their dQ atomics and Q/dO fetches meet in L2).  Workgroups are
  // dealt round-robin to the 8 XCDs: the item index is XCD-major so that all
  // items of a head share one XCD's L2.
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
  const float* Lh = NLSE + (size_t)head * N;   // -LSE / scale
  const float* Dh = NDR + (size_t)head * N;    // -D
  float* dQh = dQacc + (size_t)head * N * D;   // contiguous [B*H][N][d] accumulator

  auto run_part = [&](int part) {
    // Lane indices, re-derived per part from an opaque copy of the lane id:
    // otherwise the compiler computes lane-dependent addresses once for both
    // parts and keeps them live across the first.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int l32 = ln & 31, h = ln >> 5, g = ln >> 4, s16 = ln & 15;
    const int kb = CAUSAL ? (part == 0 ? c_item : nkb - 1 - c_item) : c_item;
    const bool ascend = part == 1;
    const int kv0 = kb * BC;
    const int kvw = kv0 + 32 * slice;        // first key row of this wave
    const int kvrow = kvw + l32;             // key row of this lane in the S accumulators
    const int krow = 32 * slice + l32;       // the same row within the block

    // dS hand-off: the wave's slice column within its head
    char* dsw = nullptr;
    if constexpr (DSO) dsw = dso.buf + (size_t)head * dso.head_bytes + (size_t)(kv0 / 32 + wave_u) * 4096u;

    // ---- K block into LDS (for K^T), then the register operands -------------
    if constexpr (DQA) {
      constexpr int KPT = BC * CH / 256;
#pragma unroll
      for (int p = 0; p < KPT; ++p) {
        const int ci = p * 256 + 64 * wave_u + ln;
        const int row = ci / CH, ch = ci % CH;
        const int kv = kv0 + row;
        u32x4 x = u32x4{0, 0, 0, 0};
        if (kv < N) x = *reinterpret_cast<const u32x4*>(Kh + (size_t)kv * lay.k.sn + ch * 8);
        *reinterpret_cast<u32x4*>(&sK[tile_off<ROWB>(row, ch)]) = x;
      }
    }
    // K_w, V_w as B operands of S = Q K^T, dP = dO V^T: lane (n = key l32, h),
    // registers d = 16*s + 8*h + r.
    bf16x8 kf[KS], vf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (kvrow < N) {
        kf[s] = *reinterpret_cast<const bf16x8*>(Kh + (size_t)kvrow * lay.k.sn + 16 * s + 8 * h);
        vf[s] = *reinterpret_cast<const bf16x8*>(Vh + (size_t)kvrow * lay.v.sn + 16 * s + 8 * h);
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
    bf16x8 ktf[DQA ? BC / 16 : 1];
    if constexpr (DQA) {
#pragma unroll
      for (int s = 0; s < BC / 16; ++s)
        ktf[s] = tr_operand<ROWB>(sK, 16 * s + 8 * h, 16 * s + 8 * h + 4, 32 * dsl + 16 * (g & 1), ln);
    }

    // ---- per-lane LDS address bases ------------------------------------------
    const TileBases<ROWB> tb(ln);
    // transposed A operand of dQ (registers = key rows) from the dS tile:
    // offset(s, u, hi) = baseE[u][hi] + 2048*s.
    int baseE[NQT][2];
    {
      const int a = s16 >> 2;
      const int E = (4 * (g & 1) + (s16 & 3)) ^ (4 * (a & 1) + 2 * h);
#pragma unroll
      for (int u = 0; u < NQT; ++u)
#pragma unroll
        for (int hi = 0; hi < 2; ++hi) {
          const int mt = mt0 + u;
          baseE[u][hi] = (8 * h + a + 4 * hi) * 128 + 64 * (mt ^ (a >> 1)) + 8 * (E ^ hi);
        }
    }

    const int i_begin = CAUSAL ? (kv0 / BR) : 0;

    // ---- direct global -> LDS fetch of one query block ------------------------
    // Q and dO tiles through TileFetch (rows past N read row N-1: finite,
    // masked later); the LSE and D rows by waves 0 and 1, 4 bytes per lane.
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

    f32x16 dk[DTW], dv[DTW];
#pragma unroll
    for (int t = 0; t < DTW; ++t) {
      dk[t] = f32x16{};
      dv[t] = f32x16{};
    }

    // dQ_ip += dS_ip K over the whole key block, from the dS tile St: the wave
    // takes d-slice dsl and query tiles mt0 .. mt0+NQT-1.  A = dS with the
    // query across lanes, B = the K^T slice in registers.
    auto dq_product = [&](int ip, const char* St) {
      if constexpr (!DQA) return;
      const int qp0 = ip * BR;
#pragma unroll
      for (int u = 0; u < NQT; ++u) {
        const int mt = mt0 + u;
        if (qp0 + 32 * mt >= N) continue;
        f32x16 acc = f32x16{};
#pragma unroll
        for (int s = 0; s < BC / 16; ++s) {
          const bf16x4 lo = lds_read_tr(St, baseE[u][0] + 2048 * s);
          const bf16x4 hi = lds_read_tr(St, baseE[u][1] + 2048 * s);
          acc = mfma32(cat(lo, hi), ktf[s], acc);
        }
        // acc[4*i4+jj] = dQ[query 32mt + 8*i4 + 4h + jj][d 32*dsl + l32]
        const int qrow0 = qp0 + 32 * mt + 4 * h;
        float* dst = dQh + (size_t)qrow0 * D + 32 * dsl + l32;
        if (qp0 + 32 * mt + 32 <= N) {
#pragma unroll
          for (int r = 0; r < 16; ++r) unsafeAtomicAdd(dst + (8 * (r >> 2) + (r & 3)) * D, acc[r]);
        } else {
          const int nvalid = N - qrow0;   // register r is a valid row iff ql(r) < nvalid
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ql = 8 * (r >> 2) + (r & 3);
            if (ql < nvalid) unsafeAtomicAdd(dst + ql * D, acc[r]);
          }
        }
      }
    };

    // Step k handles query block nqb-1-k (first part) or i_begin+k (second).
    const int nsteps = nqb - i_begin;
    // one query block: products from buffer b, prefetch into buffer b^1
    auto body = [&](auto bc, int k) {
      constexpr int b = decltype(bc)::value;
      const int i = ascend ? i_begin + k : nqb - 1 - k;
      char* Qt = b ? sQ1 : sQ0;
      char* Gt = b ? sG1 : sG0;
      const float* Lt = b ? sL1 : sL0;
      const float* Dt = b ? sD1 : sD0;
      char* St = b ? sS1 : sS0;
      const int dir = ascend ? 1 : -1;
      if (k + 1 < nsteps) fetch(i + dir, b ? sQ0 : sQ1, b ? sG0 : sG1, b ? sL0 : sL1, b ? sD0 : sD1);
      FA_DEBUG_BARRIER();
      if (k > 0) dq_product(i - dir, b ? sS0 : sS1);
      __builtin_amdgcn_sched_barrier(0);
      const int qb0 = i * BR;
      // this wave's keys are all later than all queries of the block: P^ = 0.
      // The hand-off variant runs such a step anyway (masked, it yields
      // dS = 0; the waves of a workgroup move in step, so it costs no time)
      // and stores to the sink, so that every path issues the same stores,
      // which its barrier below counts on.
      const bool dead = (kvw >= N) || (CAUSAL && qb0 + BR - 1 < kvw);
      const bool skip = DSO ? false : dead;
      // the hand-off: the BR / 16 dS micro-tiles this wave stores
      constexpr int SPW = BR / 16;
      bf16x8 dsv[SPW];
      // one pass over the block; MASK: apply the causal / tail mask (a
      // compile-time variant, so the common unmasked path carries no mask code)
      auto compute = [&](auto mc) {
        constexpr bool MASK = decltype(mc)::value;
        // P^T and dS^T as A operands (lane = key row); K-step st covers queries
        // 16st..16st+15: registers 0..3 <- 16st+4h+jj, 4..7 <- 16st+8+4h+jj.
        bf16x8 pa[BR / 16], da[BR / 16];
        // Software pipeline over the step's 32 operand groups, in this order:
        //   g = 0..7    S, dP of query tile 0, K-step g
        //   g = 8..15   S, dP of tile 1          | exponentials of tile 0
        //   g = 16..23  dV, dK of tile 0, j = g-16 | exponentials of tile 1
        //   g = 24..31  dV, dK of tile 1
        // Slot g issues the LDS reads of group g + DIST, then the two products
        // of group g, then its share of the vector work; scheduling fences
        // between slots keep this order, so each product waits only for reads
        // issued DIST slots earlier (LDS returns in order).
        // The S and dP accumulators start from -LSE/scale and -D of their
        // query rows, so they end as S - LSE/scale and dP - D.
#ifndef FA_KV_DIST
#define FA_KV_DIST 3
#endif
        constexpr int DIST = FA_KV_DIST;   // slots between an LDS read and its use
        constexpr int NG = 2 * KS + 4 * DTW;       // groups per step (4 * KS)
        // chunks of the elementwise phase of a tile: one per K-step slot
        constexpr int EC = KS;
        f32x16 s[2], dp[2];
        // dropout: per query tile, the generator of this lane quad's 4x4 block
        // in query group lane % 4 (its rounds run in the KS slots before the
        // tile's elementwise phase), then the block's bytes turned so that
        // word i holds this lane's key for query group i
        Philox4 ph[2];
        u32x4 dw[2];
        if constexpr (DROP) {
#pragma unroll
          for (int t = 0; t < 2; ++t)
            ph[t] = Philox4{(uint32_t)kvrow >> 2, (uint32_t)(qb0 + 32 * t + 8 * (ln & 3) + 4 * h) >> 2,
                            (uint32_t)head, dr.offset};
        }
        bf16x8 qa[2][KS], ga[2][KS];               // S/dP operands (Q, dO rows)
        bf16x8 tq[2][2 * DTW], tg[2][2 * DTW];     // dV/dK operands (transposed)
        auto read_group = [&](int g) {
          if (g < 2 * KS) {
            const int t = g / KS, ks = g % KS;
            const int off = tb.nat_off(t, ks);
            qa[t][ks] = lds_read_b128(Qt, off);
            ga[t][ks] = lds_read_b128(Gt, off);
          } else {
            const int t = (g - 2 * KS) / (2 * DTW), j = (g - 2 * KS) % (2 * DTW);
            const int st = 2 * t + j / DTW, dt = j % DTW;
            const int o0 = tb.tr_off(st, dt, 0), o1 = tb.tr_off(st, dt, 1);
            tg[t][j] = cat(lds_read_tr(Gt, o0), lds_read_tr(Gt, o1));
            tq[t][j] = cat(lds_read_tr(Qt, o0), lds_read_tr(Qt, o1));
          }
        };
        auto init_acc = [&](int t) {   // register r: query qb0 + 32t + 8*(r/4) + 4h + r%4
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int ql = 32 * t + 8 * i4 + 4 * h;
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(Lt + ql);
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(Dt + ql);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              s[t][4 * i4 + jj] = l4[jj];
              dp[t][4 * i4 + jj] = d4[jj];
            }
          }
        };
        auto products = [&](int g) {
          if (g < 2 * KS) {   // S = Q_i K_w^T - LSE/scale, dP = dO_i V_w^T - D
            const int t = g / KS, ks = g % KS;
            s[t] = mfma32(qa[t][ks], kf[ks], s[t]);
            dp[t] = mfma32(ga[t][ks], vf[ks], dp[t]);
          } else {            // dV += P^T dO, dK += dS^T Q
            const int t = (g - 2 * KS) / (2 * DTW), j = (g - 2 * KS) % (2 * DTW);
            const int st = 2 * t + j / DTW, dt = j % DTW;
            dv[dt] = mfma32(pa[st], tg[t][j], dv[dt]);
            dk[dt] = mfma32(da[st], tq[t][j], dk[dt]);
          }
        };
        // P^ = 2^(c (S - LSE/scale)), dS = P^ o (dP - D) for registers
        // [16 ch / EC, 16 (ch+1) / EC) of tile t (chunk ch of EC, one per slot
        // of a phase); the bf16 operands are packed once registers 0..7 and
        // 8..15 are done
        auto elem_chunk = [&](int t, int ch) {
          const int r0 = 16 * ch / EC, r1 = 16 * (ch + 1) / EC;
#pragma unroll
          for (int r = r0; r < r1; ++r) {
            float p = exp2_fast(s[t][r] * c);
            if constexpr (MASK) {
              const int q = qb0 + 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
              const bool dead = (q >= N) | (kvrow >= N) | (CAUSAL & (kvrow > q));
              p = dead ? 0.f : p;
            }
            if constexpr (DROP) {
              // -D of the register's query row, as the dP accumulator started
              const float nd = Dt[32 * t + 8 * (r >> 2) + 4 * h + (r & 3)];
              const bool keep = kept(dw[t][r >> 2], r & 3, dr.thresh);
              s[t][r] = keep ? p : 0.f;
              dp[t][r] = p * (keep ? fmaf(dr.keep_scale, dp[t][r], (1.f - dr.keep_scale) * nd) : nd);
            } else {
              s[t][r] = p;
              dp[t][r] = p * dp[t][r];
            }
          }
#pragma unroll
          for (int hi = 0; hi < 2; ++hi) {
            if (!(r0 < 8 * hi + 8 && r1 >= 8 * hi + 8)) continue;
            const int o = 8 * hi;
            pa[2 * t + hi] = pack8(s[t][o], s[t][o + 1], s[t][o + 2], s[t][o + 3],
                                   s[t][o + 4], s[t][o + 5], s[t][o + 6], s[t][o + 7]);
            da[2 * t + hi] = pack8(dp[t][o], dp[t][o + 1], dp[t][o + 2], dp[t][o + 3],
                                   dp[t][o + 4], dp[t][o + 5], dp[t][o + 6], dp[t][o + 7]);
          }
        };
        init_acc(0);
#pragma unroll
        for (int g = 0; g < DIST; ++g) read_group(g);
        init_acc(1);
        // full unrolling is required (every register array index below is a
        // compile-time constant); the dropout variant's body is past the size
        // up to which a plain unroll pragma is honoured
#pragma clang loop unroll(full)
        for (int g = 0; g < NG; ++g) {
          __builtin_amdgcn_sched_barrier(0);
          if (g + DIST < NG) read_group(g + DIST);
          products(g);
          if constexpr (DROP) {
            // tile t's rounds run in the KS slots before its elementwise phase
            if (g < 2 * KS) {
              const int t = g / KS, u = g % KS;
              ph[t].rounds(10 * u / KS, 10 * (u + 1) / KS, dr.k0, dr.k1);
              if (u == KS - 1) dw[t] = quad_transpose(byte_transpose(ph[t].words()), ln & 3);
            }
          }
          if (g >= KS && g < KS + EC) elem_chunk(0, g - KS);
          if (g >= 2 * KS && g < 2 * KS + EC) elem_chunk(1, g - 2 * KS);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (DSO) {
#pragma unroll
          for (int st = 0; st < SPW; ++st) dsv[st] = da[st];
        }
        // dS (bf16) to LDS, [key][query], for the dQ product of the atomic variant
        if constexpr (DQA) {
#pragma unroll
          for (int st = 0; st < BR / 16; ++st) {
            const bf16x4 lo = __builtin_shufflevector(da[st], da[st], 0, 1, 2, 3);
            const bf16x4 hi = __builtin_shufflevector(da[st], da[st], 4, 5, 6, 7);
            *reinterpret_cast<bf16x4*>(&St[ds_off(krow, 16 * st + 4 * h)]) = lo;
            *reinterpret_cast<bf16x4*>(&St[ds_off(krow, 16 * st + 8 + 4 * h)]) = hi;
          }
        }
      };
      if (!skip) {
        const bool need_mask = (CAUSAL && qb0 < kvw + 31) || (qb0 + BR > N) || (kvw + 32 > N);
        if (need_mask)
          compute(IC<1>{});
        else
          compute(IC<0>{});
      } else if constexpr (DQA) {
#pragma unroll
        for (int st = 0; st < BR / 16; ++st) {
          *reinterpret_cast<u32x2*>(&St[ds_off(krow, 16 * st + 4 * h)]) = u32x2{0, 0};
          *reinterpret_cast<u32x2*>(&St[ds_off(krow, 16 * st + 8 + 4 * h)]) = u32x2{0, 0};
        }
      }
      if constexpr (DSO) {
        char* p = (dead ? dso.sink : dsw + ds_block_off(CAUSAL, i, dso.nks)) + 16 * ln;
#pragma unroll
        for (int st = 0; st < SPW; ++st) __builtin_nontemporal_store(dsv[st], reinterpret_cast<bf16x8*>(p + 1024 * st));
        // s_waitcnt vmcnt(SPW) lgkmcnt(0): all but the stores (expcnt never
        // waited for).  No fence: a release fence covers the loads into LDS
        // and so waits for every memory operation; the empty asm statements
        // with a memory clobber keep the compiler from moving memory accesses
        // across the barrier.
        static_assert(SPW >= 1 && SPW <= 15, "vmcnt field");
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0x0070 | SPW);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      } else {
        __syncthreads();
      }
    };

    if (nsteps > 0) {
      fetch(ascend ? i_begin : nqb - 1, sQ0, sG0, sL0, sD0);
      __syncthreads();
      int k = 0;
      while (true) {
        body(IC<0>{}, k);
        if (++k >= nsteps) break;
        body(IC<1>{}, k);
        if (++k >= nsteps) break;
      }
      const int i_last = ascend ? nqb - 1 : i_begin;
      if (((nsteps - 1) & 1) == 0)
        dq_product(i_last, sS0);
      else
        dq_product(i_last, sS1);
    }

    // ---- write-back: dK = scale * acc, dV = acc ------------------------------
    // Each wave stages its own 32 rows through a private
    // LDS region of 32 rows (the query buffers, idle after the walk) to turn
    // the accumulator layout into 16-byte row stores.  Accumulator r of tile
    // dt: key 32*slice + 8*(r/4) + 4h + r%4, d 32*dt + l32.
    {
      char* region = (wave < 2 ? sQ0 : sG0) + (wave & 1) * (32 * ROWB);
      bf16* stg = reinterpret_cast<bf16*>(region);   // [32][D] plain row-major
      constexpr int CW = CH;                          // 16-byte chunks of a row
      constexpr int c0 = 0;                           // first column
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int dt = 0; dt < DTW; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = 8 * (r >> 2) + 4 * h + (r & 3);
            const float x = pass == 0 ? dk[dt][r] * scale : (DROP ? dv[dt][r] * dr.keep_scale : dv[dt][r]);
            stg[row * D + c0 + 32 * dt + l32] = (bf16)x;
          }
        bf16* dst = pass == 0 ? dK + lay.off(lay.dk, head) : dV + lay.off(lay.dv, head);
        const int ors = pass == 0 ? lay.dk.sn : lay.dv.sn;
        constexpr int OPW = 32 * CW / 64;   // 16-byte stores per lane
#pragma unroll
        for (int p = 0; p < OPW; ++p) {
          const int ci = p * 64 + ln;
          const int row = ci / CW, ch = ci % CW;
          if (kvw + row < N)
            *reinterpret_cast<u32x4*>(dst + (size_t)(kvw + row) * ors + c0 + ch * 8) =
                *reinterpret_cast<const u32x4*>(&stg[row * D + c0 + ch * 8]);
        }
      }
      __syncthreads();   // the next part refills the query buffers
    }
  };
  // two inlined copies rather than a loop, for the same reason
  run_part(0);
  if (nparts > 1) run_part(1);
}

template <int D, bool CAUSAL, bool DQA>
__global__ __launch_bounds__(256, 1) void bwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ NLSE, const float* __restrict__ NDR,
    float* __restrict__ dQacc, bf16* __restrict__ dK, bf16* __restrict__ dV, int BH, int N, int nqb,
    float scale, float c, Layouts lay) {
  bwd_bf16_body<D, CAUSAL, DQA, false, false>(Q, K, V, dO, NLSE, NDR, dQacc, dK, dV, BH, N, nqb, scale, c, lay,
                                              DropArgs{}, DsOut{});
}

// the same, also storing dS to the hand-off buffer
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_bf16_ds_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ NLSE, const float* __restrict__ NDR,
    bf16* __restrict__ dK, bf16* __restrict__ dV, int BH, int N, int nqb, float scale, float c, Layouts lay,
    DsOut dso) {
  bwd_bf16_body<D, CAUSAL, false, false, true>(Q, K, V, dO, NLSE, NDR, nullptr, dK, dV, BH, N, nqb, scale, c,
                                               lay, DropArgs{}, dso);
}

template <int D, bool CAUSAL, bool DSO>
__global__ __launch_bounds__(256, 1) void bwd_bf16_dropout_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ NLSE, const float* __restrict__ NDR,
    bf16* __restrict__ dK, bf16* __restrict__ dV, int BH, int N, int nqb, float scale, float c, Layouts lay,
    DropArgs dr, DsOut dso) {
  bwd_bf16_body<D, CAUSAL, false, true, DSO>(Q, K, V, dO, NLSE, NDR, nullptr, dK, dV, BH, N, nqb, scale, c, lay,
                                             dr, dso);
}

// Grid of the key/value-outer kernels: one workgroup per work item (a pair of
// key blocks when causal, one otherwise) of each head.
template <int D, bool CAUSAL>
static dim3 bwd_kv_grid(int BH, int N) {
  constexpr int BC = 128;   // keys per workgroup
  const int nkb = (N + BC - 1) / BC;
  return dim3((unsigned)((CAUSAL ? (nkb + 1) / 2 : nkb) * BH));
}

template <int D, bool CAUSAL, bool DSO>
static hipError_t launch_bwd_dropout_t(const void* q, const void* k, const void* v, const void* dO,
                                       const float* nlse, const float* ndrow, void* dk, void* dv, int BH, int N,
                                       float scale, Layouts lay, hipStream_t stream, const DropArgs& drop,
                                       DsOut ds) {
  const dim3 grid = bwd_kv_grid<D, CAUSAL>(BH, N), block(256);
  hipLaunchKernelGGL((bwd_bf16_dropout_kernel<D, CAUSAL, DSO>), grid, block, 0, stream, (const bf16*)q,
                     (const bf16*)k, (const bf16*)v, (const bf16*)dO, nlse, ndrow, (bf16*)dk, (bf16*)dv, BH, N,
                     (N + 63) / 64, scale, ledger_scale(scale) * kLog2e, lay, drop,
                     DSO ? ds : DsOut{});
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool DQA>
static hipError_t launch_bwd_bf16_t(const void* q, const void* k, const void* v, const void* dO,
                                    const float* nlse, const float* ndrow, float* dq_acc, void* dk,
                                    void* dv, int BH, int N, float scale, Layouts lay, hipStream_t stream,
                                    const DropArgs* drop, DsOut ds) {
  const int nqb = (N + 63) / 64;
  const dim3 grid = bwd_kv_grid<D, CAUSAL>(BH, N), block(256);
  const float c = ledger_scale(scale) * kLog2e;   // dK keeps the caller's scale
  if constexpr (!DQA) {
    if (drop) {
      if (ds.buf)
        return launch_bwd_dropout_t<D, CAUSAL, true>(q, k, v, dO, nlse, ndrow, dk, dv, BH, N, scale, lay, stream,
                                                     *drop, ds);
      return launch_bwd_dropout_t<D, CAUSAL, false>(q, k, v, dO, nlse, ndrow, dk, dv, BH, N, scale, lay,
                                                    stream, *drop, ds);
    }
    if (ds.buf) {
      hipLaunchKernelGGL((bwd_bf16_ds_kernel<D, CAUSAL>), grid, block, 0, stream, (const bf16*)q, (const bf16*)k,
                         (const bf16*)v, (const bf16*)dO, nlse, ndrow, (bf16*)dk, (bf16*)dv, BH, N, nqb, scale,
                         c, lay, ds);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((bwd_bf16_kernel<D, CAUSAL, DQA>), grid, block, 0, stream, (const bf16*)q,
                     (const bf16*)k, (const bf16*)v, (const bf16*)dO, nlse, ndrow, dq_acc, (bf16*)dk,
                     (bf16*)dv, BH, N, nqb, scale, c, lay);
  return hipGetLastError();
}

}  // namespace fa
