// fa_fwd_bf16.hip -- forward kernel, bf16 inputs/outputs, fp32 accumulation.
//
// One workgroup (8 waves, one workgroup per CU, two waves per SIMD) owns
// BR = 256 query rows of one (batch, head); each wave owns 32 of them (d = 256:
// 4 waves, 128 rows, one wave per SIMD).
// Key/value tiles of BC rows (64 for d = 128 and 96, 128 for d = 64, 32 for
// d = 256) stream through
// two LDS buffers (the next tile is fetched while the current one is used).
// Per tile and wave:
//   S^T = K_j Q_w^T            v_mfma_f32_32x32x16_bf16, A = K rows from LDS,
//                              B = the wave's Q rows held in registers;
//   online softmax             per lane one query row: running reference max
//                              m and running sum l, rescale factor
//                              2^(c(m_old-m_new)) when m moves (see the tile;
//                              the reference lags and moves only when needed)
//                              (page "flash-attention-v2-sram-tiling"
//                              (aiqz.cc), section 5; the l update uses the full
//                              block sum as in the derivation on page
//                              "blog.xiaohack.org/tag/flops", 知识点13 §4);
//   O^T = a O^T + V_j^T P^T    A = V^T through transposing LDS reads, B = P^T
//                              straight from the S^T accumulator registers.
// Normalisation by l is deferred to the end (the NumPy demo of page
// "flash-attention-backpropagation" (aiqz.cc), section Python 演示), and the
// ledger LSE = scale*m + ln l is written instead of P.
// The softmax runs in base 2 with the scale folded into one multiply-add:
// p = 2^(c*s - c*m) with c = scale*log2(e).  Each tile is a fixed sequence of
// slots (S products, the softmax, P V products) separated by scheduling
// fences, with the LDS operands of each slot read a few slots ahead.
//
// Split-key-range mode (SPLIT): Nq query rows against Nk >= Nq key rows (the
// decode shape), the key range of each head cut into contiguous ranges; each
// workgroup runs the same online softmax over one range for one query block
// and writes that range's O (normalised by its own l) and LSE.  The merge
// kernel then combines the ranges with the rule for joining two partial
// softmax results (page "flash-attention-v2-sram-tiling", quiz question 10).
#include "fa_common.h"
#include "fa_dropout.h"
#include "fa_launch.h"

namespace fa {

#ifndef FA_FWD_NW
#define FA_FWD_NW 8
#endif
#ifndef FA_FWD_BC64
#define FA_FWD_BC64 128
#endif
// The kernel body, shared by the plain kernel and the dropout kernel (DROP:
// the probabilities that multiply V are those of the dropout forward; the
// row sums, hence l and LSE, are those of all probabilities).
template <int D, bool CAUSAL, int NW, int BC, bool SPLIT, bool DROP>
FA_DEV void fwd_bf16_body(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
                          bf16* __restrict__ O, float* __restrict__ LSE, int BH, int N, int nqb, float scale,
                          float c, Layouts lay, SplitArgs sp, DropArgs dr) {
  static_assert(!(SPLIT && DROP), "dropout runs on the square training shape only");
  // BC: key rows per tile (128 where the registers allow it (d = 64), else 64;
  // 32 in the split mode, whose one-wave workgroups need little LDS)
  constexpr int BR = 32 * NW;
  constexpr int MT = BC / 32;        // 32-key halves of a tile
  constexpr int ROWB = lds_pitch<D>();   // LDS bytes per row (d * 2, or 256 for d = 96)
  constexpr int KS = D / 16;         // K-steps of the S product
  constexpr int DT = D / 32;         // 32-row tiles of O^T
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
  const int Nk = SPLIT ? sp.Nk : N;     // key rows
  const int off = SPLIT ? sp.off : 0;   // causal offset of the query rows
  int qb, split = 0;
  if constexpr (SPLIT) {
    split = (bid / BH) % sp.nsplit;
    qb = bid / BH / sp.nsplit;
  } else {
    // causal: the longest query blocks are dispatched first
    qb = CAUSAL ? (nqb - 1 - bid / BH) : (bid / BH);
  }
  const bf16* Qh = Q + lay.off(lay.q, head);
  const bf16* Kh = K + lay.off(lay.k, head);
  const bf16* Vh = V + lay.off(lay.v, head);

  const int q0 = qb * BR + wave * 32;   // first query row of this wave
  const int qrow = q0 + l32;            // the query row this lane's statistics belong to

  // Q rows as the B operand of S^T = K Q^T: lane (n = l32, half h) holds
  // d = 16*s + 8*h + r for K-step s.
  bf16x8 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (qrow < N)
      qf[s] = neg_bf16x8(*reinterpret_cast<const bf16x8*>(Qh + (size_t)qrow * lay.q.sn + 16 * s + 8 * h),
                         lay.qk_neg);
    else
      qf[s] = bf16x8{};
  }

  // keys of this workgroup: tiles jlo .. jlo + ntiles - 1 (all keys of the
  // head unless split), cut at the causal limit of the block's last row
  int kv_lo = 0, kv_end = Nk;
  if constexpr (SPLIT) {
    kv_lo = split * sp.span;
    kv_end = min(Nk, kv_lo + sp.span);
  }
  if (CAUSAL) kv_end = min(kv_end, qb * BR + BR + off);
  const int jlo = kv_lo / BC;
  const int ntiles = max(0, (kv_end + BC - 1) / BC - jlo);
  int wave_tiles = 0;
  if (q0 < N) {
    const int wkv_end = CAUSAL ? min(kv_end, q0 + 32 + off) : kv_end;
    wave_tiles = max(0, (wkv_end + BC - 1) / BC - jlo);
  }


  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
  float m_run = -INFINITY;   // running max of the raw scores q.k
  float l_run = 0.f;         // running sum, partial over this lane's half of the keys

  // one key/value tile: products from buffer b while tile j+1 is fetched
  // straight into buffer b^1 (distinct LDS objects per buffer, so the fetch
  // cannot alias the reads)
  auto body = [&](auto bc, int j) {
    constexpr int b = decltype(bc)::value;
    const char* Kt = b ? sK1 : sK0;
    const char* Vt = b ? sV1 : sV0;
    if (j + 1 < ntiles) {
      fetch(Kh, (jlo + j + 1) * BC, Nk, b ? sK0 : sK1);
      fetch(Vh, (jlo + j + 1) * BC, Nk, b ? sV0 : sV1, vrs);
      FA_DEBUG_BARRIER();
    }
    if (j < wave_tiles) {
      // Slots: KS slots of S products (two 32-key halves per K-step), then
      // the softmax, then (BC/16)*DT slots of P V products.  Slot i issues the
      // LDS reads of slot i + DIST before its products, with scheduling fences
      // between slots, so each product waits only for reads issued DIST slots
      // earlier (LDS returns in order).
#ifndef FA_FWD_DIST
#define FA_FWD_DIST 3
#endif
      constexpr int DIST = FA_FWD_DIST;   // slots between an LDS read and its use
      constexpr int NPV = (BC / 16) * DT;
      constexpr int NSL = KS + NPV;
      bf16x8 ka[KS][MT], vt[NPV];
      auto read_slot = [&](int i) {
        if (i < KS) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) ka[i][mt] = lds_read_b128(Kt, tb.nat_off(mt, i));
        } else {
          const int u = i - KS, st = u / DT, t = u % DT;
          vt[u] = cat(lds_read_tr(Vt, tb.tr_off(st, t, 0)), lds_read_tr(Vt, tb.tr_off(st, t, 1)));
        }
      };
      f32x16 s[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) s[mt] = f32x16{};
      bf16x8 pb[BC / 16];
      const int kvb = (jlo + j) * BC;
      // dropout: the generator for the 4x4 block of this lane's quad of query
      // rows and key group (lane % 4) of each 32-key half; its rounds run in
      // the S-product slots, which carry no other vector work
      Philox4 ph[DROP ? MT : 1];
      if constexpr (DROP) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          ph[mt] = Philox4{(uint32_t)(kvb + 32 * mt + 8 * (lane & 3) + 4 * h) >> 2, (uint32_t)qrow >> 2,
                           (uint32_t)head, dr.offset};
      }
#pragma unroll
      for (int i = 0; i < DIST; ++i) read_slot(i);
#pragma clang loop unroll(full)
      for (int i = 0; i < NSL; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (i + DIST < NSL) read_slot(i + DIST);
        if (i < KS) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) s[mt] = mfma32(ka[i][mt], qf[i], s[mt]);
          if constexpr (DROP) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) ph[mt].rounds(10 * i / KS, 10 * (i + 1) / KS, dr.k0, dr.k1);
          }
        } else {
          const int u = i - KS, st = u / DT, t = u % DT;
          oacc[t] = mfma32(vt[u], pb[st], oacc[t]);
        }
        if (i != KS - 1) continue;
        __builtin_amdgcn_sched_barrier(0);
        // s[mt][4*i+jj] = q_qrow . k_kv with kv = kvb + 32*mt + 8*i + 4*h + jj
        const bool need_mask = (kvb + BC > Nk) || (CAUSAL && kvb + BC - 1 > q0 + off);
        if (need_mask) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int kv = kvb + 32 * mt + 8 * (r >> 2) + 4 * h + (r & 3);
              const bool dead = (kv >= Nk) | (CAUSAL & (kv > qrow + off));
              s[mt][r] = dead ? -INFINITY : s[mt][r];
            }
        }
        // The probabilities are taken against a lagging reference max m_run:
        // it is moved (and O, l rescaled) only when a probability against the
        // old one could exceed 2^8, which changes nothing but the rounding (O
        // and l carry the same factor, and LSE = scale*m_run + ln l for any
        // reference).  Key 0 is never masked, so the first tile always sets
        // a finite reference; in the split mode a row may see no key of a tile
        // or of its whole range, and its reference stays -inf (no rescale,
        // p = 0) until it does.
        f32x16 sc_[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) sc_[mt] = s[mt];
        float rs = 0.f;
        auto exps = [&]() {
          const float nb = (SPLIT && m_run == -INFINITY) ? 0.f : -m_run * c;
          rs = 0.f;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float p = exp2_fast(fmaf(sc_[mt][r], c, nb));
              s[mt][r] = p;
              rs += p;
            }
        };
        auto rescale_to_max = [&](float thresh) {
          float mx = m_run;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc_[mt][r]);
          mx = half_max(mx);
          if (__builtin_amdgcn_ballot_w64((mx - m_run) * c > thresh) != 0) {
            const float alpha = (SPLIT && m_run == -INFINITY) ? 0.f : exp2_fast((m_run - mx) * c);
            l_run *= alpha;
#pragma unroll
            for (int t = 0; t < DT; ++t)
#pragma unroll
              for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;
            m_run = mx;
          }
        };
        if constexpr (SPLIT) {
          rescale_to_max(8.f);
          exps();
        } else {
          // The tile maximum is needed only when a probability could exceed
          // 2^8: first try the old reference; a lane sum above 2^8 (or not
          // finite: the first tile, against -inf) sends the wave through the
          // exact maximum and a second pass, after which every p <= 1.  A sum
          // at most 2^8 bounds every term, so the bound holds either way, and
          // the common tile skips the maximum (16 three-way max instructions
          // and a cross-lane step per lane).
          exps();
          if (__builtin_amdgcn_ballot_w64(!(rs <= 256.f)) != 0) {
            rescale_to_max(0.f);
            exps();
          }
        }
        l_run += rs;
        if constexpr (DROP) {
          // dropped probabilities leave the P V product (l keeps them)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const u32x4 w = quad_transpose(ph[mt].words(), lane & 3);
#pragma unroll
            for (int r = 0; r < 16; ++r) s[mt][r] = kept(w[r >> 2], r & 3, dr.thresh) ? s[mt][r] : 0.f;
          }
        }
        // P^T as B operand, K-step st covers keys 16*st .. 16*st+15 of the
        // tile: registers 0..3 <- keys 16st+4h+jj, 4..7 <- keys 16st+8+4h+jj
#pragma unroll
        for (int st = 0; st < BC / 16; ++st) {
          const int mt = st >> 1, i0 = 2 * (st & 1);
          pb[st] = pack8(s[mt][4 * i0 + 0], s[mt][4 * i0 + 1], s[mt][4 * i0 + 2], s[mt][4 * i0 + 3],
                         s[mt][4 * i0 + 4], s[mt][4 * i0 + 5], s[mt][4 * i0 + 6], s[mt][4 * i0 + 7]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
  };

  fetch(Kh, jlo * BC, Nk, sK0);
  fetch(Vh, jlo * BC, Nk, sV0, vrs);
  __syncthreads();
  for (int j = 0;;) {
    body(IC<0>{}, j);
    if (++j >= ntiles) break;
    body(IC<1>{}, j);
    if (++j >= ntiles) break;
  }

  if (q0 >= N) return;
  const float l_tot = half_sum(l_run);
  if constexpr (SPLIT) {
    if (qrow < N) {
      // this range's O and LSE; a row that saw no key of the range has l = 0
      const bool seen = l_tot > 0.f;
      const float inv = seen ? 1.f / l_tot : 0.f;
      const size_t prow = ((size_t)split * BH + head) * N + qrow;
      float* orow = sp.opart + prow * D;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float4 v;
          v.x = oacc[t][4 * i + 0] * inv;
          v.y = oacc[t][4 * i + 1] * inv;
          v.z = oacc[t][4 * i + 2] * inv;
          v.w = oacc[t][4 * i + 3] * inv;
          *reinterpret_cast<float4*>(orow + 32 * t + 8 * i + 4 * h) = v;
        }
      if (h == 0) sp.lpart[prow] = seen ? m_run * scale + log2_fast(l_tot) * kLn2 : -INFINITY;
    }
    return;
  }
  if (qrow < N) {
    const float inv = (DROP ? dr.keep_scale : 1.f) / l_tot;
    bf16* Orow = O + lay.off(lay.o, head) + (size_t)qrow * lay.o.sn;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x4 v;
        v[0] = (bf16)(oacc[t][4 * i + 0] * inv);
        v[1] = (bf16)(oacc[t][4 * i + 1] * inv);
        v[2] = (bf16)(oacc[t][4 * i + 2] * inv);
        v[3] = (bf16)(oacc[t][4 * i + 3] * inv);
        *reinterpret_cast<bf16x4*>(Orow + 32 * t + 8 * i + 4 * h) = v;
      }
    if (h == 0) LSE[(size_t)head * N + qrow] = m_run * scale + log2_fast(l_tot) * kLn2;
  }
}

// waves per SIMD the kernel is built for: d = 256 needs more than half the
// register file per wave (Q rows and the O accumulator alone take 192)
template <int D, int NW, bool SPLIT>
constexpr int fwd_min_blocks() {
  return SPLIT ? (D > 128 ? 1 : 2) : (D > 128 ? 4 / NW : 8 / NW);
}

template <int D, bool CAUSAL, int NW, int BC, bool SPLIT>
__global__ __launch_bounds__(64 * NW, (fwd_min_blocks<D, NW, SPLIT>())) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, int BH, int N, int nqb, float scale, float c,
    Layouts lay, SplitArgs sp) {
  fwd_bf16_body<D, CAUSAL, NW, BC, SPLIT, false>(Q, K, V, O, LSE, BH, N, nqb, scale, c, lay, sp, DropArgs{});
}

template <int D, bool CAUSAL, int NW, int BC>
__global__ __launch_bounds__(64 * NW, (fwd_min_blocks<D, NW, false>())) void fwd_bf16_dropout_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, int BH, int N, int nqb, float scale, float c,
    Layouts lay, DropArgs dr) {
  fwd_bf16_body<D, CAUSAL, NW, BC, false, true>(Q, K, V, O, LSE, BH, N, nqb, scale, c, lay, SplitArgs{}, dr);
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_bf16_t(const void* q, const void* k, const void* v, void* o, float* lse,
                                    int BH, int N, float scale, Layouts lay, hipStream_t stream,
                                    const DropArgs* drop) {
  // d = 256: 4-wave workgroups (one wave per SIMD) and 32-key tiles
  constexpr int NW = D == 256 ? 4 : FA_FWD_NW, BR = 32 * NW;
  constexpr int BC = D == 64 ? FA_FWD_BC64 : (D == 256 ? 32 : 64);
  const int nqb = (N + BR - 1) / BR;
  const dim3 grid((unsigned)(nqb * BH)), block(64 * NW);
  if (drop) {
    hipLaunchKernelGGL((fwd_bf16_dropout_kernel<D, CAUSAL, NW, BC>), grid, block, 0, stream,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, lse, BH, N, nqb, scale,
                       scale * kLog2e, lay, *drop);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, NW, BC, false>), grid, block, 0, stream,
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, lse, BH, N, nqb, scale,
                     scale * kLog2e, lay, SplitArgs{});
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                           int N, int d, bool causal, float scale, Layouts lay, hipStream_t stream,
                           const DropArgs* drop) {
  lay.qk_neg = scale < 0.f;
  scale = softmax_scale(scale);
  if (d == 128)
    return causal ? launch_fwd_bf16_t<128, true>(q, k, v, o, lse, BH, N, scale, lay, stream, drop)
                  : launch_fwd_bf16_t<128, false>(q, k, v, o, lse, BH, N, scale, lay, stream, drop);
  if (d == 256)
    return causal ? launch_fwd_bf16_t<256, true>(q, k, v, o, lse, BH, N, scale, lay, stream, drop)
                  : launch_fwd_bf16_t<256, false>(q, k, v, o, lse, BH, N, scale, lay, stream, drop);
  if (d == 96)
    return causal ? launch_fwd_bf16_t<96, true>(q, k, v, o, lse, BH, N, scale, lay, stream, drop)
                  : launch_fwd_bf16_t<96, false>(q, k, v, o, lse, BH, N, scale, lay, stream, drop);
  return causal ? launch_fwd_bf16_t<64, true>(q, k, v, o, lse, BH, N, scale, lay, stream, drop)
                : launch_fwd_bf16_t<64, false>(q, k, v, o, lse, BH, N, scale, lay, stream, drop);
}

// Split mode: one-wave workgroups of 32 query rows, 32-key tiles (16 KB of
// LDS per K/V tile pair at d = 128, so several workgroups share a CU).
template <int D, bool CAUSAL>
static hipError_t launch_fwd_split_t(const void* q, const void* k, const void* v, int BH, int Nq,
                                     float scale, Layouts lay, const SplitArgs& sp, hipStream_t stream) {
  constexpr int NW = 1, BR = 32 * NW;
  const int nqb = (Nq + BR - 1) / BR;
  const dim3 grid((unsigned)(nqb * sp.nsplit * BH)), block(64 * NW);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, NW, kSplitBC, true>), grid, block, 0, stream,
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, nullptr, nullptr, BH, Nq, nqb, scale,
                     scale * kLog2e, lay, sp);
  return hipGetLastError();
}

hipError_t launch_fwd_split_bf16(const void* q, const void* k, const void* v, float* opart, float* lpart,
                                 int BH, int Nq, int Nk, int d, bool causal, float scale, int nsplit,
                                 int span, Layouts lay, hipStream_t stream) {
  lay.qk_neg = scale < 0.f;
  scale = softmax_scale(scale);
  const SplitArgs sp{Nk, Nk - Nq, nsplit, span, opart, lpart};
  if (d == 256)
    return causal ? launch_fwd_split_t<256, true>(q, k, v, BH, Nq, scale, lay, sp, stream)
                  : launch_fwd_split_t<256, false>(q, k, v, BH, Nq, scale, lay, sp, stream);
  if (d == 128)
    return causal ? launch_fwd_split_t<128, true>(q, k, v, BH, Nq, scale, lay, sp, stream)
                  : launch_fwd_split_t<128, false>(q, k, v, BH, Nq, scale, lay, sp, stream);
  if (d == 96)
    return causal ? launch_fwd_split_t<96, true>(q, k, v, BH, Nq, scale, lay, sp, stream)
                  : launch_fwd_split_t<96, false>(q, k, v, BH, Nq, scale, lay, sp, stream);
  return causal ? launch_fwd_split_t<64, true>(q, k, v, BH, Nq, scale, lay, sp, stream)
                : launch_fwd_split_t<64, false>(q, k, v, BH, Nq, scale, lay, sp, stream);
}

}  // namespace fa
