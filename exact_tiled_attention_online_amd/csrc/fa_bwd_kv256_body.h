// fa_bwd_kv256_body.h -- the key/value-block-outer backward kernel (dK, dV) at
// d = 256, bf16 inputs/outputs, fp32 accumulation; instantiated by
// fa_bwd_kv256.hip and fa_bwd_kv256_drop.hip.
//
// The method is the one of the d <= 128 kernel (page
// "flash-attention-backpropagation" (aiqz.cc), section QKV梯度; P^ recomputed
// once per pair of blocks, page "gsyq.cn news/1372000", 踩坑二): per query
// block i and key slice w,
//   S  = Q_i K_w^T,  P^ = 2^(c*(S - LSE/scale)),   dV_w += P^T dO_i,
//   dP = dO_i V_w^T, dS = P^ o (dP - D),           dK_w += dS^T Q_i.
// What differs is how the work is split.  A 32-key slice's dK and dV over all
// 256 columns are 256 fp32 registers per lane, and its K and V rows another
// 128, more than one wave holds beside its S and dP tiles.  So two waves share
// each slice, split by product rather than by columns of d:
//  - the P wave holds the slice's K rows and one 32 x 256 accumulator, dV: it
//    forms S, P^ (masked), and dV += P^T dO over all of d;
//  - the dS wave holds the V rows and dK: it forms dP, takes P^ from the P
//    wave, forms dS and dK += dS^T Q, and (hand-off variant) stores dS.
// Every product of the method then runs once per block pair (4 of 32 x 64 x
// 256 each, one wave computing two of them), where a split by columns of d
// needs S and dP in both waves (6).  The P wave hands over P^ in fp32 through
// LDS, once per 32-query tile, with one workgroup barrier each; the dS wave
// forms dS = P^ o (dP - D) with the same operands and operations as the
// d <= 128 kernel.  A workgroup of 4 waves owns 64 keys (2 slices).
//
// Per query block the work is a fixed sequence of 64 slots separated by
// scheduling fences, one product each:
//   slots  0..15  the first product (S or dP) of query tile 0, K-step g
//   slots 16..31  the same for tile 1    | P wave: P^ of tile 0, to LDS
//                                         | dS wave: P^ of tile 0 from LDS, dS
//   slots 32..47  the second product (dV or dK) of tile 0, j = g - 32
//                                         | the same hand-over for tile 1
//   slots 48..63  the second product of tile 1
// Each slot issues the LDS reads of the slot PIPE ahead (LDS returns in
// order).  Q, dO, -LSE/scale and -D of the next query block are fetched
// straight into the other LDS buffer while the current one is used, as in the
// d <= 128 kernel (one barrier closing each block).
#pragma once
#include "fa_common.h"
#include "fa_dropout.h"
#include "fa_launch.h"

namespace fa {

namespace kv256 {
constexpr int D = 256, BC = 64, BR = 64;
constexpr int ROWB = 512, CH = D / 8, KS = D / 16, DT = D / 32;
constexpr int QTB = BR * ROWB;   // bytes of one Q or dO tile
constexpr int NG = 4 * KS;       // slots per query block: 2 tiles x (KS + 2 * DT)
// The P wave forms tile t's P^ two registers per slot in the 8 slots from
// kExp[t] (the slot after the tile's last first-product K-step), writes it to
// LDS in slot kPut[t], and meets the dS wave at a barrier in slot kTake[t]
// (two slots later, so that the writes have landed under the intervening
// slot's product); the dS wave reads it there and forms dS four registers per
// slot in the 4 slots from kDs[t], ahead of the tile's second product.
constexpr int kExp[2] = {KS, 2 * KS};
constexpr int kPut[2] = {KS + 8, 2 * KS + 8};
constexpr int kTake[2] = {KS + 10, 2 * KS + 10};
constexpr int kDs[2] = {KS + 12, 2 * KS + 12};
// LDS operand reads issued per slot g (1: natural row read; 2: two halves of a
// transposed read)
constexpr int reads_of(int g) { return g >= NG ? 0 : (g < 2 * KS ? 1 : 2); }

// The LDS of one workgroup.
struct Smem {
  char *q0, *q1, *g0, *g1;   // Q and dO tiles, two buffers each
  float *l0, *l1, *d0, *d1;  // -LSE / scale and -D of the tile's rows
  f32x4* x;                  // P^ hand-over: [slice][tile][4 register groups][64 lanes]
};
}  // namespace kv256

// One wave's part: PW selects the P wave (K, S, P^, dV) or the dS wave (V,
// dP, dS, dK).  DROP: the dropout backward (keep mask Z, keep scale s:
// dV = s (P^ o Z)^T dO, dS = P^ o (s (dP~ - D) + (s - 1) D) where kept and
// P^ o (-D) where dropped, dP~ - D being what the dP accumulator holds).
// DSO: the dS wave also stores dS to the hand-off buffer.
template <bool CAUSAL, bool DROP, bool DSO, bool PW>
FA_DEV void bwd256_wave(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
                        const bf16* __restrict__ dO, const float* __restrict__ NLSE,
                        const float* __restrict__ NDR, bf16* __restrict__ dK, bf16* __restrict__ dV, int BH,
                        int N, int nqb, float scale, float c, const Layouts& lay, const DropArgs& dr,
                        const DsOut& dso, const kv256::Smem& sm) {
  using namespace kv256;
#ifndef FA_KV_DIST
#define FA_KV_DIST 3
#endif
  // slots between an LDS read and its product: one product per slot here
  // against two in the d <= 128 kernel, so twice that kernel's distance
  constexpr int PIPE = 2 * FA_KV_DIST;
  // The Q and dO tiles are fetched by the two dS waves alone (16 loads of
  // 1 KB each per tile and wave): the P waves, whose exponentials make them
  // the longer path to each hand-over, issue no tile loads (measured 3% faster
  // than all four waves fetching).
  constexpr int NF = 2;
  static_assert(kPut[0] == kExp[0] + 8 && kPut[1] == kExp[1] + 8 && kTake[0] == kPut[0] + 2 &&
                kTake[1] == kPut[1] + 2 && kDs[0] > kTake[0] && kDs[1] > kTake[1] && kDs[0] + 4 <= 2 * KS &&
                kDs[1] + 4 <= 2 * KS + 2 * DT, "hand-over slots");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slice = wave_u >> 1;
  const TileFetch<ROWB, BR, NF, CH> qfetch(slice, lane, lay.q.sn * 2);   // Q rows; dO rows at grs (dS waves)
  const unsigned grs = (unsigned)lay.g.sn * 2u;
  // Work items as in the d <= 128 kernel: causal item c of a head is the
  // key-block pair (c, nkb-1-c), the first walked from the last query block
  // down, the second from its first query block up; items dealt XCD-major.
  const int nkb = (N + BC - 1) / BC;
  const int P = CAUSAL ? (nkb + 1) / 2 : nkb;
  const int W = P * BH;
  const int bid = blockIdx.x;
  const int item = (W % 8 == 0) ? (bid % 8) * (W / 8) + bid / 8 : bid;
  const int head = item / P, c_item = item % P;
  const int nparts = (CAUSAL && 2 * c_item + 1 != nkb) ? 2 : 1;
  const bf16* Qh = Q + lay.off(lay.q, head);
  const bf16* Gh = dO + lay.off(lay.g, head);
  const bf16* Rh = PW ? K + lay.off(lay.k, head) : V + lay.off(lay.v, head);   // the wave's operand rows
  const int rsn = PW ? lay.k.sn : lay.v.sn;
  const float* Lh = NLSE + (size_t)head * N;   // -LSE / scale
  const float* Dh = NDR + (size_t)head * N;    // -D

  for (int part = 0; part < nparts; ++part) {
    // lane indices from an opaque copy of the lane id, so that lane-dependent
    // addresses are not computed once and kept live across both parts
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int l32 = ln & 31, h = ln >> 5;
    const int kb = CAUSAL ? (part == 0 ? c_item : nkb - 1 - c_item) : c_item;
    const bool ascend = part == 1;
    const int kv0 = kb * BC;
    const int kvw = kv0 + 32 * slice;        // first key row of this wave
    const int kvrow = kvw + l32;             // key row of this lane in the accumulators

    // K_w (P wave) or V_w (dS wave) as the B operand of S = Q K^T or
    // dP = dO V^T: lane (n = key l32, h), registers d = 16*s + 8*h + r
    // (rows past N: row N-1 read, zeros kept)
    bf16x8 bop[KS];
    const bf16* rrow = Rh + (size_t)min(kvrow, N - 1) * rsn + 8 * h;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(rrow + 16 * s);
      bop[s] = kvrow < N ? v : bf16x8{};
    }

    const TileBases<ROWB> tb(ln);
    const int i_begin = CAUSAL ? (kv0 / BR) : 0;
    // Q and dO tiles through TileFetch by the dS waves (rows past N read row
    // N-1: finite, masked later); the -LSE/scale and -D rows by waves 0 and 1,
    // 4 bytes per lane
    auto fetch = [&](int i, char* dQt, char* dGt, float* dL, float* dD) {
      const int qb0 = i * BR;
      if constexpr (!PW) {
        qfetch(Qh, qb0, N, dQt);
        qfetch(Gh, qb0, N, dGt, grs);
      }
      if (qb0 + BR <= N) {
        if (wave_u == 0) dma4_buf(raw_rsrc(Lh), 4 * ln, 4 * qb0, dL);
        if (wave_u == 1) dma4_buf(raw_rsrc(Dh), 4 * ln, 4 * qb0, dD);
      } else {
        if (wave_u == 0) dma4_buf(raw_rsrc(Lh), 4 * min(qb0 + ln, N - 1), 0, dL);
        if (wave_u == 1) dma4_buf(raw_rsrc(Dh), 4 * min(qb0 + ln, N - 1), 0, dD);
      }
    };

    // dV (P wave) or dK (dS wave) of the slice: tile dt, register r holds key
    // kvw + 8*(r/4) + 4h + r%4, column 32*dt + l32
    f32x16 acc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) acc[t] = f32x16{};

    // the P^ hand-over of this slice, register group q of tile t at xs[(4t + q) * 64 + lane]
    f32x4* xs = sm.x + slice * (2 * 4 * 64);
    char* dsw = nullptr;
    if constexpr (DSO && !PW) dsw = dso.buf + (size_t)head * dso.head_bytes + (size_t)(kv0 / 32 + slice) * 4096u;

    const int nsteps = nqb - i_begin;
    auto body = [&](auto bc, int k) {
      constexpr int b = decltype(bc)::value;
      const int i = ascend ? i_begin + k : nqb - 1 - k;
      const char* Qt = b ? sm.q1 : sm.q0;
      const char* Gt = b ? sm.g1 : sm.g0;
      const float* Lt = b ? sm.l1 : sm.l0;
      const float* Dt = b ? sm.d1 : sm.d0;
      const char* T1 = PW ? Qt : Gt;          // rows of the first product's A operand
      const char* T2 = PW ? Gt : Qt;          // transposed B operand of the second product
      const float* I1 = PW ? Lt : Dt;         // start of the first product's accumulator
      const int dir = ascend ? 1 : -1;
      if (k + 1 < nsteps)
        fetch(i + dir, b ? sm.q0 : sm.q1, b ? sm.g0 : sm.g1, b ? sm.l0 : sm.l1, b ? sm.d0 : sm.d1);
      FA_DEBUG_BARRIER();
      __builtin_amdgcn_sched_barrier(0);
      const int qb0 = i * BR;
      // a slice whose keys all lie past N (a non-causal tail) runs the masked
      // step (P^ = 0); the waves of a workgroup must meet the same barriers
      const bool dead = kvw >= N;
      (void)dead;
      // dS^T (dS wave) or P^T (P wave) as A operands of the second product
      // (lane = key row): K-step st covers queries 16st..16st+15, registers
      // 0..3 <- 16st+4h+jj, 4..7 <- 16st+8+4h+jj
      bf16x8 op[BR / 16];
      // steps that need the causal or tail mask (the P wave applies it)
      const bool need_mask = (CAUSAL && qb0 < kvw + 31) || (qb0 + BR > N) || (kvw + 32 > N);
      {
        f32x16 x[2];   // S - LSE/scale then P^ (P wave), or dP - D then dS (dS wave)
        Philox4 ph[2];
        u32x4 dw[2];
        if constexpr (DROP) {
#pragma unroll
          for (int t = 0; t < 2; ++t)
            ph[t] = Philox4{(uint32_t)kvrow >> 2, (uint32_t)(qb0 + 32 * t + 8 * (ln & 3) + 4 * h) >> 2,
                            (uint32_t)head, dr.offset};
        }
        bf16x8 a1[2][KS];          // first product's A operands
        bf16x8 a2[2][2 * DT];      // second product's B operands (transposed)
        f32x4 px[2][4];            // dS wave: the P^ taken over
        auto read_group = [&](int g) {
          if (g < 2 * KS) {
            const int t = g / KS, ks = g % KS;
            a1[t][ks] = lds_read_b128(T1, tb.nat_off(t, ks));
          } else {
            const int t = (g - 2 * KS) / (2 * DT), j = (g - 2 * KS) % (2 * DT);
            const int st = 2 * t + j / DT, dt = j % DT;
            a2[t][j] = cat(lds_read_tr(T2, tb.tr_off(st, dt, 0)), lds_read_tr(T2, tb.tr_off(st, dt, 1)));
          }
        };
        // register r of tile t: query qb0 + 32t + 8*(r/4) + 4h + r%4.  On a
        // masked step the P wave starts the S accumulator of a hidden (query,
        // key) pair at the infinity whose product with c is -inf, so that its
        // P^ comes out 0 (the dot product added to it is finite): the mask
        // costs nothing on the other steps.  Hidden: query past N, key past
        // N, or (causal) key after query.
        auto init_acc = [&](int t) {
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const f32x4 v4 = *reinterpret_cast<const f32x4*>(I1 + 32 * t + 8 * i4 + 4 * h);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) x[t][4 * i4 + jj] = v4[jj];
          }
          if constexpr (PW) {
            if (need_mask) {
              // visible iff lo <= o < hi for o = q - qb0, as one unsigned test
              const int lo = kvrow >= N ? BR : (CAUSAL ? kvrow - qb0 : 0);
              const unsigned span = (unsigned)max(min(N - qb0, BR) - lo, 0);
              const float dead_s = c > 0.f ? -INFINITY : INFINITY;
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int o = 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
                x[t][r] = (unsigned)(o - lo) < span ? x[t][r] : dead_s;
              }
            }
          }
        };
        auto products = [&](int g) {
          if (g < 2 * KS) {
            const int t = g / KS, ks = g % KS;
            x[t] = mfma32(a1[t][ks], bop[ks], x[t]);
          } else {   // for each dt: K-steps 2t, 2t+1 of tile t, in the d <= 128 kernel's order
            const int t = (g - 2 * KS) / (2 * DT), j = (g - 2 * KS) % (2 * DT);
            const int st = 2 * t + j / DT, dt = j % DT;
            acc[dt] = mfma32(op[st], a2[t][j], acc[dt]);
          }
        };
        auto pack_half = [&](int t, int hi, const f32x16& v) {
          const int o = 8 * hi;
          op[2 * t + hi] = pack8(v[o], v[o + 1], v[o + 2], v[o + 3], v[o + 4], v[o + 5], v[o + 6], v[o + 7]);
        };
        // P wave, registers 2q, 2q+1 of tile t: P^; with dropout the operand
        // of dV is P^ o Z while the hand-over keeps P^
        f32x16 pz[2];   // dropout: P^ o Z, the operand of dV
        auto p_chunk = [&](int t, int q) {
#pragma unroll
          for (int r = 2 * q; r < 2 * q + 2; ++r) {
            const float p = exp2_fast(x[t][r] * c);
            x[t][r] = p;
            if constexpr (DROP) pz[t][r] = kept(dw[t][r >> 2], r & 3, dr.thresh) ? p : 0.f;
          }
          if ((q & 3) == 3) pack_half(t, q >> 2, DROP ? pz[t] : x[t]);
        };
        // dS wave, registers 4q..4q+3 of tile t: dS = P^ o (dP - D) (with
        // dropout, P^ o (s (dP~ - D) + (s - 1) D) where kept, P^ o (-D) where not)
        auto ds_chunk = [&](int t, int q) {
#pragma unroll
          for (int r = 4 * q; r < 4 * q + 4; ++r) {
            const float p = px[t][q][r & 3];
            if constexpr (DROP) {
              const float nd = Dt[32 * t + 8 * (r >> 2) + 4 * h + (r & 3)];
              const bool keep = kept(dw[t][r >> 2], r & 3, dr.thresh);
              x[t][r] = p * (keep ? fmaf(dr.keep_scale, x[t][r], (1.f - dr.keep_scale) * nd) : nd);
            } else {
              x[t][r] = p * x[t][r];
            }
          }
          if (q & 1) pack_half(t, q >> 1, x[t]);
        };
        init_acc(0);
#pragma unroll
        for (int g = 0; g < PIPE; ++g) read_group(g);
        init_acc(1);
#pragma clang loop unroll(full)
        for (int g = 0; g < NG; ++g) {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            if (g == kTake[t]) {
              // the P wave's writes of tile t are complete once at most the
              // reads issued after them (one slot's) are outstanding
              if constexpr (PW) {
                constexpr int w0 = 0xC07F | (reads_of(kPut[0] + 1 + PIPE) << 8);   // lgkmcnt(n) only
                constexpr int w1 = 0xC07F | (reads_of(kPut[1] + 1 + PIPE) << 8);
                if (t == 0)
                  __builtin_amdgcn_s_waitcnt(w0);
                else
                  __builtin_amdgcn_s_waitcnt(w1);
              }
              asm volatile("" ::: "memory");
              __builtin_amdgcn_s_barrier();
              asm volatile("" ::: "memory");
              if constexpr (!PW) {
#pragma unroll
                for (int q = 0; q < 4; ++q) px[t][q] = xs[(4 * t + q) * 64 + ln];
              }
            }
          }
          if (g + PIPE < NG) read_group(g + PIPE);
          products(g);
          if constexpr (DROP) {
            // tile t's generator rounds run in its KS first-product slots
            if (g < 2 * KS) {
              const int t = g / KS, u = g % KS;
              ph[t].rounds(10 * u / KS, 10 * (u + 1) / KS, dr.k0, dr.k1);
              if (u == KS - 1) dw[t] = quad_transpose(byte_transpose(ph[t].words()), ln & 3);
            }
          }
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            if constexpr (PW) {
              if (g >= kExp[t] && g < kPut[t]) p_chunk(t, g - kExp[t]);
              if (g == kPut[t]) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                  xs[(4 * t + q) * 64 + ln] = f32x4{x[t][4 * q], x[t][4 * q + 1], x[t][4 * q + 2], x[t][4 * q + 3]};
                // the writes stay ahead of the next slot's reads, which the
                // count at the barrier relies on
                asm volatile("" ::: "memory");
              }
            } else {
              if (g >= kDs[t] && g < kDs[t] + 4) ds_chunk(t, g - kDs[t]);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (DSO && !PW) {
        char* p = (dead ? dso.sink : dsw + ds_block_off(CAUSAL, i, dso.nks)) + 16 * ln;
#pragma unroll
        for (int st = 0; st < BR / 16; ++st)
          __builtin_nontemporal_store(op[st], reinterpret_cast<bf16x8*>(p + 1024 * st));
        // s_waitcnt vmcnt(4) lgkmcnt(0): all but the four stores (vector
        // memory operations retire in issue order, so the prefetch issued
        // before them has landed in LDS).  No fence: a release fence would
        // wait for the stores too; the empty asm statements with a memory
        // clobber keep the compiler from moving memory accesses across the
        // barrier.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0x0070 | (BR / 16));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      } else if constexpr (DSO) {
        // the P wave stores nothing: wait for everything, meet the same barrier
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0x0070);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      } else {
        __syncthreads();
      }
    };

    fetch(ascend ? i_begin : nqb - 1, sm.q0, sm.g0, sm.l0, sm.d0);
    __syncthreads();
    int k = 0;
    while (true) {
      body(IC<0>{}, k);
      if (++k >= nsteps) break;
      body(IC<1>{}, k);
      if (++k >= nsteps) break;
    }

    // ---- write-back: dV = acc (times the keep scale with dropout), dK = scale * acc
    // Each wave stages its 32 rows through a private LDS region (half of a
    // query buffer, idle after the walk) to turn the accumulator layout into
    // 16-byte row stores.
    {
      char* region = (wave_u < 2 ? sm.q0 : sm.g0) + (wave_u & 1) * (32 * ROWB);
      bf16* stg = reinterpret_cast<bf16*>(region);   // [32][D] plain row-major
      const float f = PW ? (DROP ? dr.keep_scale : 1.f) : scale;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 8 * (r >> 2) + 4 * h + (r & 3);
          stg[row * D + 32 * dt + l32] = (bf16)(PW && !DROP ? acc[dt][r] : acc[dt][r] * f);
        }
      bf16* dst = PW ? dV + lay.off(lay.dv, head) : dK + lay.off(lay.dk, head);
      const int ors = PW ? lay.dv.sn : lay.dk.sn;
      constexpr int OPW = 32 * CH / 64;   // 16-byte stores per lane
#pragma unroll
      for (int p = 0; p < OPW; ++p) {
        const int ci = p * 64 + ln;
        const int row = ci / CH, ch = ci % CH;
        if (kvw + row < N)
          *reinterpret_cast<u32x4*>(dst + (size_t)(kvw + row) * ors + ch * 8) =
              *reinterpret_cast<const u32x4*>(&stg[row * D + ch * 8]);
      }
      __syncthreads();   // the next part refills the query buffers
    }
  }
}

template <bool CAUSAL, bool DROP, bool DSO>
__global__ __launch_bounds__(256, 1) void bwd256_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ NLSE, const float* __restrict__ NDR,
    bf16* __restrict__ dK, bf16* __restrict__ dV, int BH, int N, int nqb, float scale, float c, Layouts lay,
    DropArgs dr, DsOut dso) {
  using namespace kv256;
  __shared__ __attribute__((aligned(1024))) char sQ0[QTB];
  __shared__ __attribute__((aligned(1024))) char sQ1[QTB];
  __shared__ __attribute__((aligned(1024))) char sG0[QTB];   // dO
  __shared__ __attribute__((aligned(1024))) char sG1[QTB];
  __shared__ __attribute__((aligned(256))) float sL0[BR];    // -LSE / scale
  __shared__ __attribute__((aligned(256))) float sL1[BR];
  __shared__ __attribute__((aligned(256))) float sD0[BR];    // -D
  __shared__ __attribute__((aligned(256))) float sD1[BR];
  __shared__ __attribute__((aligned(1024))) f32x4 sX[2 * 2 * 4 * 64];
  const Smem sm{sQ0, sQ1, sG0, sG1, sL0, sL1, sD0, sD1, sX};
  if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & 1)
    bwd256_wave<CAUSAL, DROP, DSO, false>(Q, K, V, dO, NLSE, NDR, dK, dV, BH, N, nqb, scale, c, lay, dr, dso, sm);
  else
    bwd256_wave<CAUSAL, DROP, DSO, true>(Q, K, V, dO, NLSE, NDR, dK, dV, BH, N, nqb, scale, c, lay, dr, dso, sm);
}

template <bool CAUSAL, bool DROP, bool DSO>
static hipError_t launch_bwd256_t(const void* q, const void* k, const void* v, const void* dO, const float* nlse,
                                  const float* ndrow, void* dk, void* dv, int BH, int N, float scale, Layouts lay,
                                  hipStream_t stream, const DropArgs& drop, DsOut ds) {
  using namespace kv256;
  const int nkb = (N + BC - 1) / BC;
  const dim3 grid((unsigned)((CAUSAL ? (nkb + 1) / 2 : nkb) * BH)), block(256);
  hipLaunchKernelGGL((bwd256_kernel<CAUSAL, DROP, DSO>), grid, block, 0, stream, (const bf16*)q, (const bf16*)k,
                     (const bf16*)v, (const bf16*)dO, nlse, ndrow, (bf16*)dk, (bf16*)dv, BH, N, (N + BR - 1) / BR,
                     scale, ledger_scale(scale) * kLog2e, lay, drop, DSO ? ds : DsOut{});
  return hipGetLastError();
}

}  // namespace fa
