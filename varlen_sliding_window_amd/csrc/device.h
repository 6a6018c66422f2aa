// Device helpers shared by the forward and backward kernels.
//
// MFMA fragment layouts used throughout (v_mfma_f32_32x32x16_bf16, one wave
// of 64 lanes, l = lane, h = l / 32, c = l % 32):
//   A (32 x 16): lane l holds A[c][8h + i], i = 0..7
//   B (16 x 32): lane l holds B[8h + i][c]
//   D (32 x 32): lane l, register r holds D[8(r/4) + 4h + (r%4)][c]
// A result's row index lives in registers and its column in the lane, so a
// result can feed the next product's reduction (k) index directly when the
// k order is permuted to match: for 16-wide step t of a 32-row result,
// element i of lane half h is row 16t + 8(i/4) + 4h + (i%4), i.e. register
// r = 8t + i.  The other operand is read in the same permuted order with two
// transposing LDS reads of 4 consecutive rows each (rows 16t + 4h + 0..3 and
// 16t + 8 + 4h + 0..3).
#pragma once

#include "common.h"

namespace attn {

__device__ __forceinline__ uint4 ldg16(const bf16* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  return __builtin_bit_cast(bf16x8, make_uint4(0u, 0u, 0u, 0u));
}

__device__ __forceinline__ f32x16 zero_f32x16() {
  f32x16 z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each block of 16 lanes,
// source lane 4i + a points at row i, columns 4a..4a+3 of a 4 x 16 bf16
// sub-matrix; destination lane 4a + b receives column 4a + b, rows 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

// ---- swizzled, unpadded LDS tiles --------------------------------------------
// A tile holds rows of D bf16 (D = 64, 128 or 256: 128, 256 or 512 bytes)
// with no padding; 16-byte chunk c of row r is stored at chunk c ^ swz<D>(r).
// The swizzle is a bijection per row (it only flips the low bits of c) and
// keeps both read patterns free of LDS bank conflicts (64 banks of 4 bytes,
// so one 256-byte line of banks):
//   16-byte row reads (16 lanes on 16 consecutive rows, same chunk): the 16
//     addresses must fall in 16 different 16-byte bank groups;
//   transposing 8-byte reads (32 lanes on 4 consecutive rows x an aligned
//     group of 4 chunks): the 4 rows must land in 4 different groups of 4.
// D = 128 (a row is one bank line): swz rotates the low four bits of r by two,
//   a bijection on 16 rows whose bits 2-3 differ within any 4 aligned rows.
// D = 256 (two bank lines per row): the same swz on the chunk's low four bits.
// D = 64 (two rows per bank line, parity picks the half): within each parity
//   class the row's bits 1-3 are rotated by one, again a bijection on the 8
//   rows of that class, and rows 4k and 4k + 2 differ in the group bit.
// Unpadded rows let one wave fill 1 KB of whole rows with a single direct
// global-to-LDS load.
template <int D>
__device__ __forceinline__ int swz(int r) {
  static_assert(D == 64 || D == 128 || D == 256, "head dims 64, 128, 256");
  if constexpr (D == 64)
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  else
    return ((r & 3) << 2) | ((r >> 2) & 3);
}

// A or B fragment whose lane index runs over rows (c = lane % 32) and whose
// register elements are 8 consecutive columns 16 ks + 8h + 0..7 of a
// swizzled tile (rows 32-aligned relative to the tile start).
template <int D>
__device__ __forceinline__ bf16x8 swz_frag_cols(const bf16* tile, int ks, int lane) {
  const int r = lane & 31;
  const int c = 2 * ks + (lane >> 5);
  return *reinterpret_cast<const bf16x8*>(tile + r * D + ((c ^ swz<D>(r)) << 3));
}

// A or B fragment whose lane index runs over 32 columns of a swizzled tile
// (starting at column col0, a multiple of 32) and whose 8 register elements
// run over rows 16t + 8(i/4) + 4h + i%4, read with two transposing reads.
template <int D>
__device__ __forceinline__ bf16x8 swz_frag_rows(const bf16* tile, int col0, int t, int lane) {
  const int r0 = 16 * t + 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int r1 = r0 + 8;
  const int col = col0 + (lane & 16) + 4 * (lane & 3);
  const int c = col >> 3, off = col & 7;
  const bf16x4 lo = lds_read_tr(tile + r0 * D + ((c ^ swz<D>(r0)) << 3) + off);
  const bf16x4 hi = lds_read_tr(tile + r1 * D + ((c ^ swz<D>(r1)) << 3) + off);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Geometry of one wave's 1 KB direct loads into a swizzled tile of rows of D
// bf16: lane l moves 16 bytes into physical chunk l % CPR of row l / CPR of
// the load's RPD rows, so it fetches the logical chunk that lands there.
template <int D>
struct TileLoad {
  static constexpr int CPR = D / 8;     // 16-byte chunks per row
  static constexpr int RPD = 64 / CPR;  // rows per 1 KB load
  // Byte offset within a row of the chunk that lane `lane` fetches, when the
  // lane lands in tile row r.
  __device__ static uint32_t chunk_offset(int lane, int r) {
    return (uint32_t)(((lane % CPR) ^ swz<D>(r)) << 4);
  }
};

// Per-head-dim geometry of the kernels that stream key-value blocks (the
// forward and dQ): 4 waves share each double-buffered K/V block in LDS.
template <int D>
struct BlockGeom {
  static constexpr int KB = D <= 128 ? 64 : 32;          // keys per block
  static constexpr int H2 = KB / 32;                     // 32-key halves of a block
  static constexpr int KS = D / 16;                      // k-steps of a D-long product
  static constexpr int DB = D / 32;                      // 32-column blocks of D
  static constexpr int TILE_BYTES = KB * D * (int)sizeof(bf16);
  static constexpr int BUF_BYTES = 2 * TILE_BYTES;       // K and V
  static constexpr int ROWS_PER_WAVE = KB / 4;           // rows each wave loads
  static constexpr int LOADS = ROWS_PER_WAVE / TileLoad<D>::RPD;   // 1 KB loads per tensor
  // work-groups per CU: 2 up to D = 128; at D = 256 a wave's operands and
  // accumulators need a whole SIMD's registers
  static constexpr int MIN_WG = D <= 128 ? 2 : 1;
  static_assert(LOADS >= 1 && ROWS_PER_WAVE % TileLoad<D>::RPD == 0, "whole loads per wave");
};

// Direct global-to-LDS load by one wave: the 16 bytes at base + off of each
// active lane land at LDS byte address lds + 16 * lane.  It is issued as
// inline assembly so that the compiler does not make later LDS reads wait
// for it: callers wait themselves (s_waitcnt vmcnt) before reading the
// destination, and never read a destination with a load still in flight.
// M0 carries the LDS address (one wait state between its write and the load)
// and is restored afterwards, since the compiler owns it.
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(base), "s"(lds)
      : "memory");
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  typedef __attribute__((address_space(3))) const char lds_cchar;
  return (uint32_t)(uintptr_t)(lds_cchar*)p;
}

// One wave's tile of 32 rows of D bf16 (a q-tile of one head) moved between
// global memory and a swizzled LDS tile with whole-row accesses: a 1 KB
// direct load or a 1 KB store per instruction, instead of 32 rows touched by
// every instruction when the rows go straight to or from MFMA fragments.
template <int D>
struct RowTile {
  static constexpr int ROWS = 32;
  static constexpr int BYTES = ROWS * D * (int)sizeof(bf16);
  static constexpr int MOVES = ROWS / TileLoad<D>::RPD;   // 1 KB moves per tile
};

// Direct loads of tile rows [0, nrows) (1 <= nrows; rows past nrows repeat row
// nrows - 1): tile row r is the global row at byte offset r * stride_b from
// base.  The caller waits (s_waitcnt vmcnt) before reading the tile.
template <int D>
__device__ __forceinline__ void dma_tile_rows(const bf16* base, uint32_t stride_b, int nrows,
                                              uint32_t lds, int lane) {
#pragma unroll
  for (int j = 0; j < RowTile<D>::MOVES; ++j) {
    const int r = TileLoad<D>::RPD * j + lane / TileLoad<D>::CPR;
    const uint32_t off = (uint32_t)min(r, nrows - 1) * stride_b + TileLoad<D>::chunk_offset(lane, r);
    dma16(base, off, lds + j * 1024);
  }
}

// Writes the wave's accumulator fragments acc[db] (lane l: row l % 32,
// columns 32 db + 8(i/4) + 4(l/32) + i%4, see the D layout above), times
// `scale`, as bf16 into a swizzled 32 x D LDS tile.
template <int D>
__device__ __forceinline__ void stage_acc_rows(bf16* tile, const f32x16* acc, float scale,
                                               int lane) {
  const int row = lane & 31, half = lane >> 5;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 4 * db + j;
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (bf16)(acc[db][4 * j + e] * scale);
      *reinterpret_cast<bf16x4*>(tile + row * D + ((c ^ swz<D>(row)) << 3) + 4 * half) = v;
    }
}

// Stores tile rows [0, nrows) of a swizzled 32 x D LDS tile to global rows
// `stride` elements apart starting at base, 16 bytes per lane.  The tile is
// the wave's own (LDS operations of one wave complete in order).
template <int D>
__device__ __forceinline__ void store_tile_rows(bf16* base, size_t stride, int nrows,
                                                const bf16* tile, int lane) {
#pragma unroll
  for (int j = 0; j < RowTile<D>::MOVES; ++j) {
    const int r = TileLoad<D>::RPD * j + lane / TileLoad<D>::CPR;
    const int c = lane % TileLoad<D>::CPR;
    const uint4 v = *reinterpret_cast<const uint4*>(tile + r * D + ((c ^ swz<D>(r)) << 3));
    if (r < nrows) *reinterpret_cast<uint4*>(base + (size_t)r * stride + c * 8) = v;
  }
}

// Writes `word` to every 4-byte word of [p, p + nwords), spread over all
// work-groups of the launch: the outputs of a call whose schedule does not
// belong to it, or whose boundaries are malformed, become NaN.
constexpr uint32_t NAN_BF16X2 = 0x7FC07FC0u;   // two bf16 quiet NaNs
constexpr uint32_t NAN_F32 = 0x7FC00000u;
__device__ __forceinline__ void poison_words(void* p, size_t nwords, uint32_t word) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  uint32_t* w = static_cast<uint32_t*>(p);
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords; i += stride)
    w[i] = word;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// max(x of lane l, x of lane l ^ 32): the two lanes that hold one query row's
// halves of a 32 x 32 accumulator.  v_permlane32_swap hands each lane both
// x[l % 32] and x[l % 32 + 32] in registers, without the LDS round trip of a
// shuffle.
__device__ __forceinline__ float row_halves_max(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// tanh in fp32 with a relative error of about 2e-7 everywhere.
//   |x| >= 0.55: 1 - 2 / (exp(2x) + 1) from the hardware exp2 and reciprocal;
//     a large x makes the exponential +inf and the quotient 0 (tanh = 1), a
//     very negative one makes it 0 (tanh = -1).
//   |x| <  0.55: x + x^3 g(x^2), where the quartic g was fitted by weighted
//     least squares to (tanh(x) - x) / x^3 on that interval; the exponential
//     form would lose all relative accuracy as x -> 0 (a cap far above the
//     logits then still reproduces them).
constexpr float TANH_NARROW = 0.55f;   // |x| below this takes the polynomial

__device__ __forceinline__ float tanh_narrow(float x) {
  const float y = x * x;
  float g = -0.00636491494f;
  g = fmaf(g, y, 0.0211331641f);
  g = fmaf(g, y, -0.0538665094f);
  g = fmaf(g, y, 0.133327132f);
  g = fmaf(g, y, -0.33333321f);
  return fmaf(x * y, g, x);
}

__device__ __forceinline__ float tanh_fast(float x) {
  const float wide = 1.f - 2.f * __builtin_amdgcn_rcpf(exp2_fast(x * (2.f * LOG2E)) + 1.f);
  return fabsf(x) < TANH_NARROW ? tanh_narrow(x) : wide;
}

// Soft-capped logits of M accumulator fragments, in place: x <- tanh(a x).
// When no lane of the wave holds an argument outside the polynomial's range
// (the usual case for a cap well above the logits) the exponential form is
// not evaluated at all.  `thr` = TANH_NARROW / a.
template <int M>
__device__ __forceinline__ void tanh_fragments(f32x16* x, float a, float thr) {
  float big = 0.f;
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) big = fmaxf(big, fabsf(x[m][i]));
  if (__builtin_amdgcn_ballot_w64(!(big < thr))) {   // NaN takes the general path
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int i = 0; i < 16; ++i) x[m][i] = tanh_fast(a * x[m][i]);
  } else {
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int i = 0; i < 16; ++i) x[m][i] = tanh_narrow(a * x[m][i]);
  }
}

__device__ __forceinline__ void store_bf16x4(bf16* p, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (bf16)a;
  v[1] = (bf16)b;
  v[2] = (bf16)c;
  v[3] = (bf16)d;
  *reinterpret_cast<bf16x4*>(p) = v;
}

}  // namespace attn
