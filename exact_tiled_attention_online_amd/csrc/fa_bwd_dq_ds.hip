// fa_bwd_dq_ds.hip -- dQ = scale * dS K from the dS hand-off buffer, bf16 out,
// fp32 accumulation.
//
// dQ_i = scale * sum_j dS_ij K_j (page "flash-attention-backpropagation"
// (aiqz.cc), section QKV梯度), with dS exactly the bf16 operand the
// key/value-outer kernel formed from its single recompute of P^ (page "gsyq.cn
// news/1372000", 踩坑二: one recompute feeds all three gradients).  No S or dP
// product is repeated and no atomics are used: the work per (query, key) pair
// is one product, and the kernel is bound by reading dS (2 bytes per pair).
//
// One workgroup (4 waves) owns 128 query rows of one (batch, head): query
// blocks 2I and 2I+1 of 64 rows, each wave a 32-row half of one block, with
// dQ^T (d x 32) in registers.  It walks the keys in stages of 64 (two 32-key
// slices of the buffer) through LDS, K one stage ahead, dS (the HBM stream)
// two stages ahead:
//   K stage       64 rows, swizzled tile, fetched by all four waves
//   dS stage      per wave, the two 1 KB micro-tiles (16 queries each) of its
//                 32 queries for each of the two slices
// and per 16-key step
//   dQ^T += K^T dS^T     MFMA, A = K^T and B = dS^T, both through transposing
//                        LDS reads (lane = d column, resp. query; registers =
//                        keys, in the same order on both sides).
// A micro-tile holds lane (key + 32h)'s 16 bytes (queries 16st + 4h + 0..3,
// then 16st + 8 + 4h + 0..3).  It lands in LDS through non-temporal buffer
// loads straight into LDS (each byte is read once; measured 9% faster than
// cached loads), lane l fetching 16-byte chunk l ^ 4*bit5(l) ^ 8*u (u: the
// micro-tile's position within the 32 queries), so that the 32 lanes of a
// transposing read (4 keys x 16 queries, two micro-tiles) hit 32 distinct
// 8-byte bank slots.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dq_ds_kernel(const char* __restrict__ dsbuf, size_t ds_head_bytes,
                                                            int nks, const bf16* __restrict__ K,
                                                            bf16* __restrict__ dQ, int BH, int N, int nqb,
                                                            float scale, Layouts lay) {
  constexpr int ROWB = lds_pitch<D>();   // LDS bytes per K row (d * 2, or 256 for d = 96)
  constexpr int DT = D / 32;             // 32-row tiles of dQ^T
  constexpr int KC = 64;                 // keys per stage
  constexpr int KTB = KC * ROWB;         // bytes of a K stage
  constexpr int WSB = 4096;              // dS bytes of a stage per wave (2 slices x 2 micro-tiles)
  // K stages double-buffered (fetched one stage ahead), dS stages in three
  // buffers (fetched two stages ahead: dS is the stream from HBM)
  __shared__ __attribute__((aligned(1024))) char sK0[KTB];
  __shared__ __attribute__((aligned(1024))) char sK1[KTB];
  __shared__ __attribute__((aligned(1024))) char sS0[4 * WSB];
  __shared__ __attribute__((aligned(1024))) char sS1[4 * WSB];
  __shared__ __attribute__((aligned(1024))) char sS2[4 * WSB];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, g = lane >> 4, s16 = lane & 15;
  const int l32 = lane & 31;
  const int nI = (nqb + 1) / 2;   // 128-row work items per head
  const int bid = blockIdx.x;
  const int head = bid % BH;
  // causal: the longest items are dispatched first
  const int I = CAUSAL ? nI - 1 - bid / BH : bid / BH;
  const int b = 2 * I + (wave >> 1);   // this wave's 64-row query block
  const int qt = wave & 1;             // its 32-row half of the block
  const bool has_blk = b < nqb;
  // 32-key slices stored for a block (the buffer's layout)
  auto slices = [&](int blk) { return CAUSAL ? min(2 * blk + 2, nks) : nks; };
  const int nsl_w = has_blk ? slices(b) : 0;
  const int nstage = (slices(min(2 * I + 1, nqb - 1)) + 1) / 2;
  const bf16* Kh = K + lay.off(lay.k, head);
  const TileFetch<ROWB, KC, 4, D / 8> kfetch(wave, lane, lay.k.sn * 2);
  const TileBases<ROWB> tb(lane);

  // the wave's block in the buffer (block 0 of the head for a wave without
  // one: its fetches below stay in bounds and are never read); slice ks of it
  // sits ks * 4 KB further
  const __amdgpu_buffer_rsrc_t rs =
      raw_rsrc(dsbuf + (size_t)head * ds_head_bytes + ds_block_off(CAUSAL, has_blk ? b : 0, nks));
  const int last_sl = max(nsl_w, 1) - 1;   // fetches of slices past the block's re-read its last one
  unsigned voff[2];   // micro-tile 2qt + u: the chunk this lane fetches
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int ch = lane ^ (((lane >> 5) & 1) << 2) ^ (u << 3);
    voff[u] = (unsigned)(1024 * (2 * qt + u) + 16 * ch);
  }
  // transposing reads of dS^T: lane (g, s16) points at key kk = 16*kk2 + 4h +
  // 8*hi + s16/4 of the slice, queries 4a .. 4a+3 (a = s16 % 4) of micro-tile
  // u = g % 2, i.e. byte 8*(a/2) of chunk kk + 32*(a%2), placed as above
  int boff[2][2];
  {
    const int u = g & 1, a = s16 & 3;
#pragma unroll
    for (int kk2 = 0; kk2 < 2; ++kk2)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int kk = 16 * kk2 + 4 * h + 8 * hi + (s16 >> 2);
        const int pos = (kk + 32 * (a & 1)) ^ (4 * (a & 1)) ^ (8 * u);
        boff[kk2][hi] = 1024 * u + 16 * pos + 8 * (a >> 1);
      }
  }

  // Every fetch call issues the same loads on every path (stages past the
  // end re-read the last one, slices past the wave's block re-read its last
  // slice), so that the wait closing each stage can count them: the four dS
  // loads of the newest fetch are the only ones it leaves outstanding.
  auto fetch_k = [&](int s, char* Kt) { kfetch(Kh, KC * min(s, nstage - 1), N, Kt); };
  auto fetch_ds = [&](int s, char* St) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int ks = min(2 * s + j, last_sl);
#pragma unroll
      for (int u = 0; u < 2; ++u)   // non-temporal (aux bit 1): dS is read once
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (FA_LDS void*)(St + wave * WSB + (2 * j + u) * 1024), 16, voff[u],
                                                 (unsigned)ks * 4096u, 0, 2);
    }
  };
  // s_waitcnt vmcnt(4) lgkmcnt(0), then the barrier; no fence (a release
  // fence covers the loads into LDS and so waits for all of them), empty asm
  // statements with a memory clobber keep memory accesses on their side
  auto stage_barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0074);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  f32x16 acc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) acc[t] = f32x16{};

  // stage s: products from K buffer s % 2 and dS buffer s % 3, while K of
  // stage s+1 and dS of stage s+2 are fetched into the buffers stage s-1 used.
  // All of the stage's operands are read from LDS before those fetches are
  // issued (80 registers), so that no read waits for a load issued after it
  // (the compiler cannot tell the fetch targets apart from the buffers read).
  auto body = [&](auto kc, auto sc, int s) {
    constexpr int kb = decltype(kc)::value, sb = decltype(sc)::value;
    const char* Kt = kb ? sK1 : sK0;
    const char* St = (sb == 0 ? sS0 : (sb == 1 ? sS1 : sS2)) + wave * WSB;
    bf16x8 bop[4], aop[4][DT];
#pragma unroll
    for (int kst = 0; kst < 4; ++kst) {
      const int j = kst >> 1;
      if (2 * s + j < nsl_w) {
        const char* Sj = St + 2048 * j;
        bop[kst] = cat(lds_read_tr(Sj, boff[kst & 1][0]), lds_read_tr(Sj, boff[kst & 1][1]));
#pragma unroll
        for (int t = 0; t < DT; ++t)
          aop[kst][t] = cat(lds_read_tr(Kt, tb.tr_off(kst, t, 0)), lds_read_tr(Kt, tb.tr_off(kst, t, 1)));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    fetch_k(s + 1, kb ? sK0 : sK1);
    fetch_ds(s + 2, sb == 0 ? sS2 : (sb == 1 ? sS0 : sS1));
    FA_DEBUG_BARRIER();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kst = 0; kst < 4; ++kst) {
      if (2 * s + (kst >> 1) < nsl_w) {
#pragma unroll
        for (int t = 0; t < DT; ++t) acc[t] = mfma32(aop[kst][t], bop[kst], acc[t]);
      }
    }
    stage_barrier();
  };

  fetch_k(0, sK0);
  fetch_ds(0, sS0);
  fetch_ds(1, sS1);
  stage_barrier();
  for (int s = 0;;) {
    body(IC<0>{}, IC<0>{}, s);
    if (++s >= nstage) break;
    body(IC<1>{}, IC<1>{}, s);
    if (++s >= nstage) break;
    body(IC<0>{}, IC<2>{}, s);
    if (++s >= nstage) break;
    body(IC<1>{}, IC<0>{}, s);
    if (++s >= nstage) break;
    body(IC<0>{}, IC<1>{}, s);
    if (++s >= nstage) break;
    body(IC<1>{}, IC<2>{}, s);
    if (++s >= nstage) break;
  }
  // the fetches past the end must land before the workgroup's LDS goes
  __builtin_amdgcn_s_waitcnt(0x0070);

  const int qrow = 64 * b + 32 * qt + l32;
  if (!has_blk || qrow >= N) return;
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

template <int D, bool CAUSAL>
static hipError_t launch_dq_ds_t(DsOut ds, const void* k, void* dq, int BH, int N, float scale, Layouts lay,
                                 hipStream_t stream) {
  const int nqb = (N + 63) / 64, nI = (nqb + 1) / 2;
  const dim3 grid((unsigned)(nI * BH)), block(256);
  hipLaunchKernelGGL((bwd_dq_ds_kernel<D, CAUSAL>), grid, block, 0, stream, (const char*)ds.buf, ds.head_bytes,
                     ds.nks, (const bf16*)k, (bf16*)dq, BH, N, nqb, scale, lay);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_ds(DsOut ds, const void* k, void* dq, int BH, int N, int d, bool causal, float scale,
                            Layouts lay, hipStream_t stream) {
  auto go = [&](auto dc) {
    constexpr int D = decltype(dc)::value;
    return causal ? launch_dq_ds_t<D, true>(ds, k, dq, BH, N, scale, lay, stream)
                  : launch_dq_ds_t<D, false>(ds, k, dq, BH, N, scale, lay, stream);
  };
  if (d == 128) return go(IC<128>{});
  if (d == 256) return go(IC<256>{});
  if (d == 96) return go(IC<96>{});
  return go(IC<64>{});
}

}  // namespace fa
