// fa_fwd_fp8.hip -- forward kernel with FP8 (OCP e4m3fn) Q, K, V and per-tensor
// descales; O in bf16, LSE in fp32.
//
// The method is the forward of fa_fwd_bf16.hip (online softmax, page
// "flash-attention-v2-sram-tiling" (aiqz.cc), section 5; deferred
// normalisation as in the NumPy demo of page
// "flash-attention-backpropagation", section Python 演示), with both products
// on gfx950's FP8 matrix instruction v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3
// operands, unit block scales, fp32 accumulation), which does twice the work
// per cycle of the bf16 one.  The FP8 forward of FlashAttention-3 is the
// variant the pages name (page "data.6616ai.com flash-attention"); this is a
// gfx950 design of it.
//
// Values: Q = descale_q * Q8 and so on, so S = (scale * descale_q * descale_k)
// * (Q8 K8^T) and O = descale_v * softmax(S) V8.  The dot products of e4m3
// codes are exact in fp32, so S and the softmax statistics (m, l, LSE) are as
// accurate as in the bf16 kernel.  P is rounded to e4m3 for the P V product:
// each probability is taken as p * 2^7 <= 2^8 (the reference maximum moves
// whenever a row's maximum grows by more than a factor 2^1), which keeps it
// below the e4m3 limit of 448 and above the subnormal range for every p that
// matters; l sums the same scaled values in fp32, so the factor cancels in
// O = sum(P V) / l and LSE subtracts 7 ln 2.
//
// Work split: one workgroup (4 waves) owns 128 query rows of one (batch, head),
// each wave 32, and three workgroups share a CU (three waves per SIMD: the
// softmax's vector work, which bounds this kernel, then overlaps the products
// of other waves more often than with two); key/value tiles of 64 rows of 128
// bytes stream through two LDS buffers.  Per tile and wave:
//   S^T (2 x 32 keys x 32 queries): A = K rows (natural 16-byte LDS reads),
//       B = the wave's Q rows in registers; 2 K-steps of 64 d;
//   O^T += V^T P^T, one K-step of all 64 keys: B = P^T packed to e4m3
//       straight from the S^T accumulators (lane = query, 32 keys per lane),
//       A = V^T gathered by the 8-bit transposing LDS read in the same key
//       order as B.
// Operand layout of the FP8 instruction: lane l holds row (or column) l % 32
// and 32 consecutive K-values of group l / 32; any assignment of K-values to
// bytes works as long as A and B use the same one, which is how P^T (in the
// accumulator's key order) meets V^T.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4v __attribute__((ext_vector_type(4)));
typedef int i32x2v __attribute__((ext_vector_type(2)));

// e4m3 x e4m3 (format code 0 for A and B), unit E8M0 block scales (127 = 2^0)
FA_DEV f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

FA_DEV i32x4v lds_read_i128(const char* base, int off) {
  return *reinterpret_cast<const i32x4v*>(base + off);
}

// 8-bit transposing read: in each group of 16 lanes, lane 8u + c receives
// byte c of the 8-byte segments addressed by lanes 2e + u, e = 0..7, as its
// bytes e (measured on the device).
FA_DEV i32x2v lds_read_tr8(const char* base, int off) {
  typedef FA_LDS i32x2v lds_i32x2;
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(base + off));
}

FA_DEV i32x8 cat8(i32x4v a, i32x4v b) { return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7); }

FA_DEV i32x8 cat_tr(i32x2v a, i32x2v b, i32x2v c, i32x2v d) {
  const i32x4v lo = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const i32x4v hi = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return cat8(lo, hi);
}

// four e4m3 codes of four floats in one dword (round to nearest even).  The
// first conversion writes the low half and keeps the high half of its third
// operand, which the second conversion then overwrites; passing a's own bits
// there (a dies here) lets the result take a's register, where a constant 0
// cost one register initialisation per dword.
FA_DEV int pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

#ifndef FA_FP8_NW
#define FA_FP8_NW 4
#endif
// NW waves per workgroup; at about 160 VGPRs three waves fit per SIMD, so
// three 4-wave workgroups share a CU.  SPLIT: the split-key-range mode of the
// bf16 forward (Nq queries against Nk keys, one range of whole tiles per
// workgroup, partial O and LSE to the workspace for the merge kernel).
template <int D, bool CAUSAL, int NW, bool SPLIT>
__global__ __launch_bounds__(64 * NW, D == 256 ? 1 : (SPLIT ? 2 : 12 / NW)) void fwd_fp8_kernel(
    const unsigned char* __restrict__ Q, const unsigned char* __restrict__ K,
    const unsigned char* __restrict__ V, bf16* __restrict__ O, float* __restrict__ LSE, int BH, int N,
    int nqb, float scale_qk, float c, float dv, Layouts lay, SplitArgs sp) {
  static_assert(D == 64 || D == 96 || D == 128 || D == 256, "FP8 head dims");
  constexpr int BR = 32 * NW, BC = 64;
  // LDS rows are 128 bytes up to d = 128 (the 128-byte swizzle) and 256 bytes
  // at d = 256 (the 256-byte swizzle); d = 64 and 96 fill 4 and 6 of their 8
  // chunks, and the fetch points the other lanes at a row's last chunk (in
  // bounds, finite, multiplied by zeros below).  Every offset of 16 or 32
  // rows is a multiple of ROWB (the swizzles depend on the row mod 16 only).
  constexpr int ROWB = D <= 128 ? 128 : 256;
  constexpr int KS = (D + 63) / 64;  // K-steps of 64 d of the S product
  constexpr int DT = D / 32;         // 32-row tiles of O^T
  constexpr int TILEB = BC * ROWB;   // bytes of one K or V tile

  __shared__ __attribute__((aligned(1024))) char sK0[TILEB];
  __shared__ __attribute__((aligned(1024))) char sK1[TILEB];
  __shared__ __attribute__((aligned(1024))) char sV0[TILEB];
  __shared__ __attribute__((aligned(1024))) char sV1[TILEB];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5;
  // strides in elements (= bytes for the e4m3 inputs)
  const TileFetch<ROWB, BC, NW, D / 16> fetch(wave, lane, lay.k.sn);   // K rows; V rows at vrs
  const unsigned vrs = (unsigned)lay.v.sn;
  const int bid = blockIdx.x;
  const int head = bid % BH;
  const int Nk = SPLIT ? sp.Nk : N;     // key rows
  const int off = SPLIT ? sp.off : 0;   // causal offset of the query rows
  int qb, split = 0;
  if constexpr (SPLIT) {
    split = (bid / BH) % sp.nsplit;
    qb = bid / BH / sp.nsplit;
  } else {
    qb = CAUSAL ? (nqb - 1 - bid / BH) : (bid / BH);   // longest blocks first
  }
  const unsigned char* Qh = Q + lay.off(lay.q, head);
  // TileFetch moves bytes; it takes the tile base as a bf16 pointer
  const bf16* Kh = reinterpret_cast<const bf16*>(K + lay.off(lay.k, head));
  const bf16* Vh = reinterpret_cast<const bf16*>(V + lay.off(lay.v, head));

  const int q0 = qb * BR + wave * 32;
  const int qrow = q0 + l32;

  // Q rows as B operands: lane (query l32, group h) holds d = 64s + 32h .. +31;
  // zeros past d (d = 96: the second K-step's upper half), so that the
  // padding chunks of the K tiles add nothing to S
  i32x8 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (qrow < N && 64 * s + 32 * h < D) {
      const i32x4v* p = reinterpret_cast<const i32x4v*>(Qh + (size_t)qrow * lay.q.sn + 64 * s + 32 * h);
      // a negative scale: the sign bit of every e4m3 code flipped (exact)
      const int m = lay.qk_neg ? (int)0x80808080u : 0;
      qf[s] = cat8(p[0], p[1]) ^ i32x8{m, m, m, m, m, m, m, m};
    } else {
      qf[s] = i32x8{};
    }
  }

  // LDS offsets.  K operand (key row l32 of a 32-key half, bytes 64s + 32h ..
  // +31 as two 16-byte chunks): kb[s][hf] + 32 * ROWB * half (swz depends on the
  // row mod 16, so 32 rows down is a constant).
  int kb[KS][2];
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) kb[s][hf] = tile_off<ROWB>(l32, 4 * s + 2 * h + hf);
  // V^T operand for the 32 d-rows 32t .. 32t+31: four transposing reads w;
  // this lane supplies the segment of key row 16w + r0 (r0 as below), bytes
  // 32t + 16(G%2) + 8u .. +7, so that the receiving lane (d, group g) gets,
  // as its bytes 8w + e, V[key 16w + 8(e/4) + 4g + e%4][d]: the key order of
  // the P^T operand.  Offset vb[t] + 16 * ROWB * w.
  int vb[DT];
  {
    const int G = (lane >> 4) & 3, e = (lane & 15) >> 1, u = lane & 1;
    const int r0 = 8 * (e >> 2) + 4 * (G >> 1) + (e & 3);
#pragma unroll
    for (int t = 0; t < DT; ++t) vb[t] = r0 * ROWB + (((2 * t + (G & 1)) ^ swz<ROWB>(r0)) << 4) + 8 * u;
  }

  // keys of this workgroup: tiles jlo .. jlo + ntiles - 1
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
  float m_run = -INFINITY;   // reference maximum of the raw code dot products
  float l_run = 0.f;         // sum of 2^7 p, partial over this lane's half of the keys

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
      // Slots: KS slots of two S products (the two 32-key halves), the
      // softmax, DT slots of one P V product; each slot first issues the LDS
      // reads of the slot DIST ahead.
      constexpr int DIST = 2;
      constexpr int NSL = KS + DT;
      i32x8 ka[KS][2], va[DT];
      auto read_slot = [&](int i) {
        if (i < KS) {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
            ka[i][mt] = cat8(lds_read_i128(Kt, kb[i][0] + 32 * ROWB * mt),
                             lds_read_i128(Kt, kb[i][1] + 32 * ROWB * mt));
        } else {
          const int t = i - KS;
          va[t] = cat_tr(lds_read_tr8(Vt, vb[t]), lds_read_tr8(Vt, vb[t] + 16 * ROWB),
                         lds_read_tr8(Vt, vb[t] + 32 * ROWB), lds_read_tr8(Vt, vb[t] + 48 * ROWB));
        }
      };
      f32x16 s[2] = {f32x16{}, f32x16{}};
      i32x8 pb;
      const int kvb = (jlo + j) * BC;
#pragma unroll
      for (int i = 0; i < DIST; ++i) read_slot(i);
#pragma clang loop unroll(full)
      for (int i = 0; i < NSL; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (i + DIST < NSL) read_slot(i + DIST);
        if (i < KS) {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) s[mt] = mfma_fp8(ka[i][mt], qf[i], s[mt]);
        } else {
          oacc[i - KS] = mfma_fp8(va[i - KS], pb, oacc[i - KS]);
        }
        if (i != KS - 1) continue;
        __builtin_amdgcn_sched_barrier(0);
        // s[mt][4*r4+jj] = q8_qrow . k8_kv with kv = kvb + 32*mt + 8*r4 + 4*h + jj
        const bool need_mask = (kvb + BC > Nk) || (CAUSAL && kvb + BC - 1 > q0 + off);
        if (need_mask) {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int kv = kvb + 32 * mt + 8 * (r >> 2) + 4 * h + (r & 3);
              const bool dead = (kv >= Nk) | (CAUSAL & (kv > qrow + off));
              s[mt][r] = dead ? -INFINITY : s[mt][r];
            }
        }
        float mx = m_run;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mt][r]);
        mx = half_max(mx);
        // as in the bf16 forward, the reference maximum moves (with O and l
        // rescaled) only when a row gains more than a factor 2^1 over it, so
        // that 2^7 p stays at most 2^8 < 448 (split mode: a row that has seen
        // no key yet keeps -inf, no rescale and p = 0, as in the bf16 forward)
        if (__builtin_amdgcn_ballot_w64((mx - m_run) * c > 1.f) != 0) {
          const float alpha = (SPLIT && m_run == -INFINITY) ? 0.f : exp2_fast((m_run - mx) * c);
          l_run *= alpha;
#pragma unroll
          for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;
          m_run = mx;
        }
        const float nb = (SPLIT && m_run == -INFINITY) ? 7.f : 7.f - m_run * c;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[mt][r] = exp2_fast(fmaf(s[mt][r], c, nb));
        // the tile's sum as a tree (31 adds, no chain through a zero start)
        float part[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) part[r] = s[0][r] + s[1][r];
#pragma unroll
        for (int w = 8; w > 0; w >>= 1)
#pragma unroll
          for (int r = 0; r < w; ++r) part[r] += part[r + w];
        l_run += part[0];
        // P^T as the B operand: byte 16*mt + r of this lane (query qrow,
        // group h) is the key kvb + 32*mt + 8*(r/4) + 4*h + r%4
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            pb[4 * mt + q] = pack_fp8x4(s[mt][4 * q], s[mt][4 * q + 1], s[mt][4 * q + 2], s[mt][4 * q + 3]);
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
      const float f = seen ? dv / l_tot : 0.f;
      const size_t prow = ((size_t)split * BH + head) * N + qrow;
      float* orow = sp.opart + prow * D;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float4 x;
          x.x = oacc[t][4 * i + 0] * f;
          x.y = oacc[t][4 * i + 1] * f;
          x.z = oacc[t][4 * i + 2] * f;
          x.w = oacc[t][4 * i + 3] * f;
          *reinterpret_cast<float4*>(orow + 32 * t + 8 * i + 4 * h) = x;
        }
      if (h == 0) sp.lpart[prow] = seen ? m_run * scale_qk + (log2_fast(l_tot) - 7.f) * kLn2 : -INFINITY;
    }
    return;
  }
  if (qrow < N) {
    const float f = dv / l_tot;
    bf16* Orow = O + lay.off(lay.o, head) + (size_t)qrow * lay.o.sn;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x4 v;
        v[0] = (bf16)(oacc[t][4 * i + 0] * f);
        v[1] = (bf16)(oacc[t][4 * i + 1] * f);
        v[2] = (bf16)(oacc[t][4 * i + 2] * f);
        v[3] = (bf16)(oacc[t][4 * i + 3] * f);
        *reinterpret_cast<bf16x4*>(Orow + 32 * t + 8 * i + 4 * h) = v;
      }
    if (h == 0) LSE[(size_t)head * N + qrow] = m_run * scale_qk + (log2_fast(l_tot) - 7.f) * kLn2;
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_fp8_t(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                                   int N, float scale_qk, float dv, Layouts lay, hipStream_t stream) {
  constexpr int NW = FA_FP8_NW, BR = 32 * NW;
  const int nqb = (N + BR - 1) / BR;
  const dim3 grid((unsigned)(nqb * BH)), block(64 * NW);
  hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL, NW, false>), grid, block, 0, stream, (const unsigned char*)q,
                     (const unsigned char*)k, (const unsigned char*)v, (bf16*)o, lse, BH, N, nqb, scale_qk,
                     scale_qk * kLog2e, dv, lay, SplitArgs{});
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N, int d,
                          bool causal, float scale, float dq, float dk, float dv, Layouts lay,
                          hipStream_t stream) {
  lay.qk_neg = scale < 0.f;
  const float scale_qk = softmax_scale(fabsf(scale) * dq * dk);
  auto go = [&](auto dc) {
    constexpr int D = decltype(dc)::value;
    return causal ? launch_fwd_fp8_t<D, true>(q, k, v, o, lse, BH, N, scale_qk, dv, lay, stream)
                  : launch_fwd_fp8_t<D, false>(q, k, v, o, lse, BH, N, scale_qk, dv, lay, stream);
  };
  if (d == 64) return go(IC<64>{});
  if (d == 96) return go(IC<96>{});
  if (d == 256) return go(IC<256>{});
  return go(IC<128>{});
}

// Split mode: one-wave workgroups of 32 query rows against one key range of
// whole 64-key tiles (32 KB of LDS), partial results to the workspace.
template <int D, bool CAUSAL>
static hipError_t launch_fwd_split_fp8_t(const void* q, const void* k, const void* v, int BH, int Nq,
                                         float scale_qk, float dv, Layouts lay, const SplitArgs& sp,
                                         hipStream_t stream) {
  const int nqb = (Nq + 31) / 32;
  const dim3 grid((unsigned)(nqb * sp.nsplit * BH)), block(64);
  hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL, 1, true>), grid, block, 0, stream, (const unsigned char*)q,
                     (const unsigned char*)k, (const unsigned char*)v, nullptr, nullptr, BH, Nq, nqb, scale_qk,
                     scale_qk * kLog2e, dv, lay, sp);
  return hipGetLastError();
}

hipError_t launch_fwd_split_fp8(const void* q, const void* k, const void* v, float* opart, float* lpart,
                                int BH, int Nq, int Nk, int d, bool causal, float scale, float dq, float dk,
                                float dv, int nsplit, int span, Layouts lay, hipStream_t stream) {
  const SplitArgs sp{Nk, Nk - Nq, nsplit, span, opart, lpart};
  lay.qk_neg = scale < 0.f;
  const float scale_qk = softmax_scale(fabsf(scale) * dq * dk);
  auto go = [&](auto dc) {
    constexpr int D = decltype(dc)::value;
    return causal ? launch_fwd_split_fp8_t<D, true>(q, k, v, BH, Nq, scale_qk, dv, lay, sp, stream)
                  : launch_fwd_split_fp8_t<D, false>(q, k, v, BH, Nq, scale_qk, dv, lay, sp, stream);
  };
  if (d == 64) return go(IC<64>{});
  if (d == 96) return go(IC<96>{});
  if (d == 256) return go(IC<256>{});
  return go(IC<128>{});
}

}  // namespace fa
