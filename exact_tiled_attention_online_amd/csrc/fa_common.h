// fa_common.h -- gfx950 building blocks shared by the attention kernels:
// MFMA wrappers, the swizzled LDS tile layout, transposing LDS reads and
// wave-half exchanges.  CDNA4 only (wave64, v_mfma_*_bf16 with K=16/32,
// ds_read_b64_tr_b16, v_permlane32_swap).
//
// Register layouts (checked on the device against a host matmul):
//   v_mfma_f32_32x32x16_bf16  A: lane l holds row m = l%32, k = 8*(l/32)+r
//                             B: lane l holds col n = l%32, k = 8*(l/32)+r
//                             C: lane l, reg 4*i+j holds row 8*i+4*(l/32)+j,
//                                col l%32  (i, j in 0..3)
// The contraction index k may be permuted freely as long as A and B agree,
// which is how C tiles are reused as the next product's operand without a
// round trip: a C tile holds its N index across lanes and its M index in
// registers, exactly what an A or B operand wants for (lane = M or N,
// registers = K).
//
// ds_read_b64_tr_b16: within each 16-lane group, if lane s points at the
// 4-element row segment M[k0 + s/4][n0 + 4*(s%4) .. +3] of a row-major bf16
// tile, lane i receives the column slice M[k0 .. k0+3][n0 + i].  This gives
// an operand whose registers run down a row-major tile's rows (the
// transposed read every K-major operand needs).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))
#define FA_DEV __device__ __forceinline__

namespace fa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

FA_DEV f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

FA_DEV float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
FA_DEV float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Combine a per-lane value with the value of lane l^32 (the other wave half).
FA_DEV float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
FA_DEV float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- swizzled row-major tiles in LDS -----------------------------------
// The LDS of gfx950 serves 256 bytes per clock as 64 four-byte banks: a
// 16-byte read (ds_read_b128) is served 16 lanes at a time, an 8-byte
// transposing read 32 lanes at a time (measured with the bank-conflict
// counter).  A tile of rows of ROWB bytes (ROWB = 128, 256 or 512) is stored as
// 16-byte chunks, chunk c of row r at chunk position c ^ swz(r):
//   ROWB = 256: swz(r) = 4*(r%4) + (r/4)%4
//   ROWB = 128: swz(r) = 4*((r/2)%2) + (r/4)%4
// so that both the operand reads (16 consecutive rows at one chunk) and the
// transposing reads (4 consecutive rows, first a multiple of 4, times 4
// consecutive chunks, first a multiple of 4) touch 16 distinct 16-byte bank
// groups.  swz(r) depends on r % 16 only.  512-byte rows (d = 256) take the
// 256-byte swizzle: it leaves bit 4 of the chunk index alone, so chunks
// 16..31 sit 256 bytes after chunks 0..15 in the same bank groups.
template <int ROWB>
FA_DEV int swz(int r) {
  if constexpr (ROWB >= 256) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

template <int ROWB>
FA_DEV int tile_off(int row, int chunk) {
  return row * ROWB + ((chunk ^ swz<ROWB>(row)) << 4);
}
// byte offset of element (row, col) (bf16 columns) in the swizzled tile
template <int ROWB>
FA_DEV int tile_off_elem(int row, int col) {
  return tile_off<ROWB>(row, col >> 3) + ((col & 7) << 1);
}

FA_DEV bf16x8 lds_read_b128(const char* base, int off) {
  return *reinterpret_cast<const bf16x8*>(base + off);
}

FA_DEV bf16x4 lds_read_tr(const char* base, int off) {
  typedef FA_LDS i16x4 lds_i16x4;
  // generic -> LDS address-space cast of a pointer into a __shared__ array
  lds_i16x4* p = (lds_i16x4*)(base + off);
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
  return __builtin_bit_cast(bf16x4, v);
}

FA_DEV bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Transposed operand (8 K-values per lane) from a swizzled row-major tile
// whose rows are the K index: two 4-row tr reads, rows k0..k0+3 and
// k1..k1+3, at the 16-column group n0 (lane group g = lane/16 supplies the
// columns n0 .. n0+15, the caller folds g into n0).
template <int ROWB>
FA_DEV bf16x8 tr_operand(const char* tile, int k0, int k1, int n0, int lane) {
  const int s = lane & 15;
  const int col = n0 + 4 * (s & 3);
  const bf16x4 lo = lds_read_tr(tile, tile_off_elem<ROWB>(k0 + (s >> 2), col));
  const bf16x4 hi = lds_read_tr(tile, tile_off_elem<ROWB>(k1 + (s >> 2), col));
  return cat(lo, hi);
}

// Per-lane bases that turn every operand access of a swizzled tile into
// base + compile-time offset, so that only a handful of address registers
// stay live.  swz(row) depends on row % 16 only, so moving by a multiple of
// 16 rows adds a constant; the chunk-dependent parts get one base each.
template <int ROWB>
struct TileBases {
  static constexpr int KS = ROWB / 32;   // 16-wide K-steps per row
  static constexpr int DT = ROWB / 64;   // 32-column groups per row
  // Chunks 16 and up sit 256 bytes after chunks 0..15 (the swizzle only
  // touches the low 4 bits of the chunk index), so 512-byte rows need no more
  // bases than 256-byte ones: KSB, DTB bases plus compile-time offsets.
  static constexpr int KSB = KS < 8 ? KS : 8;
  static constexpr int DTB = DT < 4 ? DT : 4;
  // natural operand (lane = row 32*t + l32, registers = 8 elements of chunk
  // 2*ks + h):  off(t, ks) = nat[ks % KSB] + 256*(ks / KSB) + 32*t*ROWB
  int nat[KSB];
  // transposed operand (lane = column 32*t + 16*(g%2) + s, registers = rows
  // k0..k0+3 and k0+8..k0+11 with k0 = 16*st + 4*h):
  // off(st, t, hi) = tr[t % DTB][hi] + 256*(t / DTB) + 16*st*ROWB
  int tr[DTB][2];
  FA_DEV TileBases(int lane) {
    const int l32 = lane & 31, h = lane >> 5, g = lane >> 4, s16 = lane & 15;
#pragma unroll
    for (int ks = 0; ks < KSB; ++ks) nat[ks] = tile_off<ROWB>(l32, 2 * ks + h);
#pragma unroll
    for (int t = 0; t < DTB; ++t)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi)
        tr[t][hi] = tile_off_elem<ROWB>(4 * h + (s16 >> 2) + 8 * hi, 32 * t + 16 * (g & 1) + 4 * (s16 & 3));
  }
  FA_DEV int nat_off(int t, int ks) const { return nat[ks % KSB] + 256 * (ks / KSB) + 32 * t * ROWB; }
  FA_DEV int tr_off(int st, int t, int hi) const { return tr[t % DTB][hi] + 256 * (t / DTB) + 16 * st * ROWB; }
};

template <int B>
using IC = std::integral_constant<int, B>;

// FA_DEBUG_SYNC (a checking build, libfa_debug_sync.so): a full workgroup
// barrier (every memory operation of every wave complete) right after each
// prefetch of a next tile is issued, so that the prefetch has landed before
// the current tile's reads begin and no wave runs ahead into a buffer another
// wave still reads.  Its results must be bit-identical to the normal build's;
// a difference points at a missing wait or barrier around an LDS buffer swap.
#ifdef FA_DEBUG_SYNC
#define FA_DEBUG_BARRIER() __syncthreads()
#else
#define FA_DEBUG_BARRIER() \
  do {                      \
  } while (0)
#endif


// Wave-wide direct fetch global -> LDS through a buffer resource: lane l's 16
// (or 4) bytes, read from base + soffset (uniform) + voffset (per lane), land
// at lds_base + 16*l (or 4*l); lds_base must be the same for the whole wave.
// A uniform block offset thus costs no vector arithmetic.  Only the buffer
// (MUBUF) form is used: the compiler treats a pending global_load_lds (a FLAT
// instruction) as possibly out of order with LDS reads and then waits for
// every outstanding LDS read at each use, which defeats reading operands ahead.
// The resource covers the whole 32-bit range (callers stay in bounds).
FA_DEV __amdgpu_buffer_rsrc_t raw_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, -1, 0x00020000);
}
FA_DEV void dma16_buf(__amdgpu_buffer_rsrc_t rs, unsigned voff, unsigned soff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (FA_LDS void*)lds_base, 16, voff, soff, 0, 0);
}
FA_DEV void dma4_buf(__amdgpu_buffer_rsrc_t rs, unsigned voff, unsigned soff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (FA_LDS void*)lds_base, 4, voff, soff, 0, 0);
}

// LDS row pitch (bytes) of a tile of D-wide bf16 rows.  The swizzles above
// cover 128-, 256- and 512-byte rows; the 192-byte rows of d = 96 sit in
// 256-byte slots, whose chunks 12..15 hold no data (and are never read).
template <int D>
constexpr int lds_pitch() {
  return D * 2 <= 128 ? 128 : (D * 2 <= 256 ? 256 : 512);
}

// Fetch ROWS rows (VC 16-byte chunks each in global memory, rsb bytes apart)
// starting at row0 of a bf16 matrix into a swizzled LDS tile of ROWB-byte
// rows (VC <= ROWB/16), with the NW waves of a workgroup.  Wave w,
// load j fills LDS bytes [(w*LPW + j) KB, +1 KB): tile row blk*RPL + lane/CH
// at chunk position lane%CH, i.e. logical chunk (lane%CH) ^ swz(row).  Rows at
// or past nrows read row nrows-1 instead (finite values the caller masks);
// lanes whose chunk is past the row's VC chunks read its last chunk again
// (their LDS slots are padding).
// The per-lane byte offsets within a tile do not depend on row0, so they are
// computed once; a whole tile is then fetched from a uniform base address plus
// those offsets, and only a ragged last tile takes the clamped per-row path.
template <int ROWB, int ROWS, int NW = 4, int VC = ROWB / 16>
struct TileFetch {
  static constexpr int CH = ROWB / 16, RPL = 1024 / ROWB, LPW = ROWS / RPL / NW;
  static_assert(LPW * RPL * NW == ROWS, "tile must split evenly over the waves");
  unsigned goff[LPW];   // byte offset of this lane's chunk from the tile's first row
  int wave, lane;       // wave: uniform across the wave
  unsigned rsb;         // bytes between consecutive rows in global memory
  FA_DEV TileFetch(int wave_, int lane_, int row_stride_bytes)
      : wave(wave_), lane(lane_), rsb((unsigned)row_stride_bytes) {
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int row = (wave * LPW + j) * RPL + lane / CH;
      const int ch = min((lane % CH) ^ swz<ROWB>(row), VC - 1);
      goff[j] = (unsigned)row * rsb + (unsigned)(ch * 16);
    }
  }
  FA_DEV void operator()(const bf16* src, int row0, int nrows, char* dst) const {
    if (row0 + ROWS <= nrows) {
      const __amdgpu_buffer_rsrc_t rs = raw_rsrc(src);
      const unsigned soff = (unsigned)row0 * rsb;
#pragma unroll
      for (int j = 0; j < LPW; ++j) dma16_buf(rs, goff[j], soff, dst + (wave * LPW + j) * 1024);
    } else {
      ragged(src, row0, nrows, dst, rsb);
    }
  }
  // The same for a matrix whose rows are rsb2 bytes apart.  Its per-lane
  // offsets are this fetcher's moved by row * (rsb2 - rsb): one lane term and
  // one uniform term per load instead of a second set of offsets (registers
  // the callers do not have).  The wrapping 32-bit sums are exact, since every
  // true offset is below 2^31.
  FA_DEV void operator()(const bf16* src, int row0, int nrows, char* dst, unsigned rsb2) const {
    if (row0 + ROWS <= nrows) {
      const __amdgpu_buffer_rsrc_t rs = raw_rsrc(src);
      const unsigned delta = rsb2 - rsb;
      const unsigned lane_shift = (unsigned)(lane / CH) * delta;
      const unsigned soff = (unsigned)row0 * rsb2;
#pragma unroll
      for (int j = 0; j < LPW; ++j)
        dma16_buf(rs, goff[j] + lane_shift + (unsigned)((wave * LPW + j) * RPL) * delta, soff,
                  dst + (wave * LPW + j) * 1024);
    } else {
      ragged(src, row0, nrows, dst, rsb2);
    }
  }
  // a tile reaching past nrows: per-row clamped offsets
  FA_DEV void ragged(const bf16* src, int row0, int nrows, char* dst, unsigned stride) const {
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int blk = wave * LPW + j;
      const int row = blk * RPL + lane / CH;
      const int ch = min((lane % CH) ^ swz<ROWB>(row), VC - 1);
      const int r = min(row0 + row, nrows - 1);
      dma16_buf(raw_rsrc(src), (unsigned)r * stride + (unsigned)(ch * 16), 0, dst + blk * 1024);
    }
  }
};

// x with the sign of every element flipped when neg (uniform), else x: the
// sign of a negative scale folded into a bf16 operand (exact).
FA_DEV bf16x8 neg_bf16x8(bf16x8 x, int neg) {
  const uint32_t m = neg ? 0x80008000u : 0u;
  return __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, x) ^ u32x4{m, m, m, m});
}

FA_DEV bf16x8 pack8(float a0, float a1, float a2, float a3, float b0, float b1, float b2, float b3) {
  bf16x8 r;
  r[0] = (bf16)a0; r[1] = (bf16)a1; r[2] = (bf16)a2; r[3] = (bf16)a3;
  r[4] = (bf16)b0; r[5] = (bf16)b1; r[6] = (bf16)b2; r[7] = (bf16)b3;
  return r;
}

}  // namespace fa
