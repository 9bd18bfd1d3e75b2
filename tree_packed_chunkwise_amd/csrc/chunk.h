// chunk.h -- chunk-local building blocks shared by the fused forward and the
// reverse kernels (gfx950, 512 threads = 8 waves per block).
//
// Matrix-core formats used:
//   * v_mfma_f32_16x16x32_bf16 on hi/lo-split operands (hi = bf16(x),
//     lo = bf16(x - hi); product hi*hi + hi*lo + lo*hi) for the decay-factored
//     products A and P, whose factors span a wide exponent range.
//   * v_mfma_f32_16x16x32_f16, one pass, for the state products, and
//     v_mfma_f32_16x16x16_f16 for the 16x16 blocks of the triangular solves
//     (operand magnitudes are bounded, and fp16 keeps 11 mantissa bits).
//   Each hi/lo product keeps about 16 mantissa bits; a single bf16 rounding
//   per operand would cost about 1.6e-3 relative error by itself.
//
// Register-resident operands.  A 16x16 fp32 accumulator tile gives lane l the
// rows 4(l/16)..4(l/16)+3 of column l%16.  Two vertically adjacent tiles,
// converted to fp16, are therefore a valid 32-deep B fragment when the k
// index of lane group g = l/16 runs over {4g..4g+3, 16+4g..16+4g+3}; the A
// fragment (read from LDS) uses the same k order.  This keeps the recurrent
// state and the per-chunk delta in registers across every product of a chunk.
//
// Decay factors: e^(Gam_i - Gam_j) (j <= i) is split around a reference m per
// 16-row block pair (I, J) as e^(Gam_i - m) e^(m - Gam_j), m = Gam at the
// first row of block J.  The left factor is <= 1; the right one is bounded by
// the decay from the first row of block J to row j.  The reference never lies
// after either row of the pair, so an output row depends only on the rows up
// to it: a chunk shared by two trajectories up to a fork gives the same bits
// before the fork in both.
//
// Any gate g <= 0 is supported.  A row j whose decay from its block's first
// row exceeds kExactDecay in some channel would push the right factor out of
// the range where the split keeps its precision (and past fp32 from about
// 88).  From the first such row of a chunk on, every row's A and P entries
// are recomputed pair by pair with exact exponentials e^(Gam_i - Gam_j) <= 1
// (chunk_AP_exact).  Which rows take that path is decided by the rows up to
// them, so the causal property above still holds.
#pragma once

#include "common.h"

namespace kda {

constexpr int NT = 512;  // threads per block
constexpr int NW = 8;    // waves per block
// largest decay (Gam at a block's first row minus Gam at a later row of the
// block) that the factored products take; rows past it use exact pairs
constexpr float kExactDecay = 64.f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// hi = bf16(x), lo = bf16(x - hi)
__device__ inline void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = (__bf16)x;
  lo = (__bf16)(x - (float)hi);
}
// The same split of two values at once, in the packed form the conversions
// produce (element 0 in the low half): one packed conversion for the high
// parts, whose values come back by shift and mask, the exact remainders, one
// packed conversion for the low parts.  Identical results to split_bf16.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ inline void split_bf16x2(float x0, float x1, bf16x2& hi, bf16x2& lo) {
  hi = __builtin_convertvector((f32x2){x0, x1}, bf16x2);
  const unsigned hb = __builtin_bit_cast(unsigned, hi);
  const float h0 = __uint_as_float(hb << 16), h1 = __uint_as_float(hb & 0xffff0000u);
  lo = __builtin_convertvector((f32x2){x0 - h0, x1 - h1}, bf16x2);
}
// eight values of hi/lo splits, from four pairs
__device__ inline bf16x8 join8(const bf16x2& a, const bf16x2& b, const bf16x2& c, const bf16x2& d) {
  return __builtin_shufflevector(__builtin_shufflevector(a, b, 0, 1, 2, 3),
                                 __builtin_shufflevector(c, d, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
}
// hi/lo splits of eight values
__device__ inline void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
  bf16x2 h[4], l[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) split_bf16x2(x[2 * p], x[2 * p + 1], h[p], l[p]);
  hi = join8(h[0], h[1], h[2], h[3]);
  lo = join8(l[0], l[1], l[2], l[3]);
}

__device__ inline f32x4 mfma16(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ inline f32x4 mfmab(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x4 mfma16k16(const f16x4& a, const f16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ inline f16x4 acc4(const f32x4& t) {
  f16x4 r;
  r[0] = (_Float16)t[0]; r[1] = (_Float16)t[1]; r[2] = (_Float16)t[2]; r[3] = (_Float16)t[3];
  return r;
}

// Sum over the 16 lanes of a row (lanes 16r .. 16r+15) with DPP moves: quad
// swaps (xor 1, xor 2), then the half-row and row mirrors.  Every lane of the
// row ends with the same value (each step adds a commutative pair), in a
// fixed order.  VALU only: no LDS round trips, unlike a lane shuffle.
template <int CTRL>
__device__ inline float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, false));
}
__device__ inline float row_sum16(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);  // row_half_mirror
  x += dpp_mov<0x140>(x);  // row_mirror
  return x;
}

// Sums of 16 values over the 16 lanes of a row at once: a butterfly of DPP
// moves (row mirror, half-row mirror, quad swaps) in which each step keeps
// half of the values and sends the other half to the partner lane.  Lane l
// of the row returns sum over the row's lanes of x[l].
__device__ inline float row_reduce16x16(const float (&x)[16]) {
  const int i = threadIdx.x & 15;
  float y8[8], y4[4], y2[2];
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const bool hi = i & 8;
    y8[n] = (hi ? x[8 + n] : x[n]) + dpp_mov<0x140>(hi ? x[n] : x[8 + n]);
  }
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const bool hi = i & 4;
    y4[n] = (hi ? y8[4 + n] : y8[n]) + dpp_mov<0x141>(hi ? y8[n] : y8[4 + n]);
  }
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const bool hi = i & 2;
    y2[n] = (hi ? y4[2 + n] : y4[n]) + dpp_mov<0x4E>(hi ? y4[n] : y4[2 + n]);
  }
  const bool hi = i & 1;
  return (hi ? y2[1] : y2[0]) + dpp_mov<0xB1>(hi ? y2[0] : y2[1]);
}

// 4x4 transpose over the lanes of each DPP quad: afterwards lane 4a + b
// holds in x[j] what lane 4a + j held in x[b].  Two exchange stages (lane
// distance 2, then 1), each sending half of the values to the partner lane.
//
// Its use: an MFMA accumulator lane (l16 = 4a + b, g) holds rows R + 4g + r,
// r = 0..3, of column c0 + l16; after the transpose it holds row R + 4g + b,
// columns c0 + 4a .. c0 + 4a + 3, a contiguous piece of a row-major tile that
// one vector load or store moves (quad_row / quad_col below).
__device__ inline void quad_transpose(float (&x)[4]) {
  const int b = threadIdx.x & 3;
  {
    const bool hi = b & 2;
    const float r0 = dpp_mov<0x4E>(hi ? x[0] : x[2]);  // quad_perm [2,3,0,1]
    const float r1 = dpp_mov<0x4E>(hi ? x[1] : x[3]);
    if (hi) { x[0] = r0; x[1] = r1; } else { x[2] = r0; x[3] = r1; }
  }
  {
    const bool odd = b & 1;
    const float r0 = dpp_mov<0xB1>(odd ? x[0] : x[1]);  // quad_perm [1,0,3,2]
    const float r1 = dpp_mov<0xB1>(odd ? x[2] : x[3]);
    if (odd) { x[0] = r0; x[2] = r1; } else { x[1] = r0; x[3] = r1; }
  }
}
__device__ inline void quad_transpose(f32x4& v) {
  float x[4] = {v[0], v[1], v[2], v[3]};
  quad_transpose(x);
  v = (f32x4){x[0], x[1], x[2], x[3]};
}
// row offset (within a 16-row block) and column offset (within a 16-column
// block) of this lane's piece after quad_transpose
__device__ inline int quad_row() { return 4 * ((threadIdx.x & 63) >> 4) + (threadIdx.x & 3); }
__device__ inline int quad_col() { return threadIdx.x & 12; }

// four consecutive input elements (bf16 bits or fp32), one vector load
template <typename TIn>
using in4_t = TIn __attribute__((ext_vector_type(4)));
__device__ inline f32x4 in4_to_f32(const in4_t<float>& v) { return v; }
__device__ inline f32x4 in4_to_f32(const in4_t<uint16_t>& v) {
  return (f32x4){__uint_as_float((unsigned)v[0] << 16), __uint_as_float((unsigned)v[1] << 16),
                 __uint_as_float((unsigned)v[2] << 16), __uint_as_float((unsigned)v[3] << 16)};
}
// store four floats as fp16 (8 bytes) / load four fp16 as floats
__device__ inline void st_h4(_Float16* p, const f32x4& v) {
  *(f16x4*)p = (f16x4){(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
}
__device__ inline f32x4 ld_h4(const _Float16* p) {
  const f16x4 h = *(const f16x4*)p;
  return (f32x4){(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
}
// The tiles that pass between the library's own kernels (the fp16 chunk
// start states and end-state gradients, the chunk-row gradients dy, the
// per-chunk dO, the V of a chunk image) are kept as 16x16 tiles in matrix-core
// accumulator order: tile (C, W) holds rows 16C .. 16C + 15 and columns
// 16W .. 16W + 15 at elements (C (D/16) + W) 256, and inside it lane
// l = l16 + 16 g of the wave that carries column block W keeps what a 16x16
// accumulator tile gives it, rows 16C + 4g .. 16C + 4g + 3 of column
// 16W + l16, at 4 l .. 4 l + 3.  One wave's store or load of a tile thus
// moves 512 (fp16) or 1024 (fp32) contiguous bytes, and neither the writer
// nor a reader that works in accumulator layout moves values between lanes.
template <int D>
__device__ inline size_t state_tile(int C, int W) {
  return (size_t)(C * (D / 16) + W) * 256 + 4 * (threadIdx.x & 63);
}
// element offset of (row i, column c) of a [*][D] matrix kept in such tiles
template <int D>
__device__ inline size_t tile_elem(int i, int c) {
  return (size_t)((i >> 4) * (D / 16) + (c >> 4)) * 256 + 4 * ((c & 15) + 16 * ((i & 15) >> 2)) + (i & 3);
}

// B fragment from two accumulator tiles (rows 0-15 and 16-31 of a 32-deep k step)
__device__ inline f16x8 acc_pair(const f32x4& t0, const f32x4& t1) {
  f16x8 r;
  r[0] = (_Float16)t0[0]; r[1] = (_Float16)t0[1]; r[2] = (_Float16)t0[2]; r[3] = (_Float16)t0[3];
  r[4] = (_Float16)t1[0]; r[5] = (_Float16)t1[1]; r[6] = (_Float16)t1[2]; r[7] = (_Float16)t1[3];
  return r;
}
__device__ inline f16x8 acc_half(const f32x4& t0) {
  f16x8 r;
  r[0] = (_Float16)t0[0]; r[1] = (_Float16)t0[1]; r[2] = (_Float16)t0[2]; r[3] = (_Float16)t0[3];
  r[4] = r[5] = r[6] = r[7] = (_Float16)0.f;
  return r;
}

// A fragment in register k order: row `row` of an fp16 [*][pitch] array,
// k = kb + {4g..4g+3, 16+4g..16+4g+3}; `half_only` zeroes the second half
// (a k step wider than the contraction).
__device__ inline f16x8 lds_a_perm(const _Float16* base, int pitch, int row, int kb, int g,
                                   bool half_only = false) {
  const _Float16* p = base + row * pitch + kb + 4 * g;
  const f16x4 lo = *(const f16x4*)p;
  f16x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  if (half_only) {
    r[4] = r[5] = r[6] = r[7] = (_Float16)0.f;
  } else {
    const f16x4 hi = *(const f16x4*)(p + 16);
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  }
  return r;
}

// Fragments of X^T from a 16-bit row-major LDS array X[*][pitch] with the
// transposing read ds_read_b64_tr_b16: within each 16-lane group, lane l gets
// element l % 4 of the 8-byte chunk addressed by lane 4 e + l / 4, e = 0..3.
// If lane s of group g addresses X[r0 + 4 g + s / 4][c0 + 4 (s % 4)], lane
// (l16, g) receives X[r0 + 4 g + e][c0 + l16]: the 16x16x16 fragment of X^T
// with rows c0 .. c0+15 and k = r0 + 4 g + e.  c0 and the pitch are multiples
// of 4 halves (8-byte aligned chunks).
__device__ inline f16x4 lds_tr4(const _Float16* X, int pitch, int r0, int c0) {
  typedef short s16x4_t __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63, s = lane & 15, g = lane >> 4;
  const _Float16* p = X + (r0 + 4 * g + (s >> 2)) * pitch + c0 + 4 * (s & 3);
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)p);
  return __builtin_bit_cast(f16x4, v);
}
// 32-deep A fragment of X^T in register k order (rows c0 + l16 of X^T, k =
// r0 + {4g..4g+3, 16+4g..16+4g+3}); `half_only` zeroes the second half.
__device__ inline f16x8 lds_a_perm_tr(const _Float16* X, int pitch, int r0, int c0,
                                      bool half_only = false) {
  const f16x4 lo = lds_tr4(X, pitch, r0, c0);
  f16x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  if (half_only) {
    r[4] = r[5] = r[6] = r[7] = (_Float16)0.f;
  } else {
    const f16x4 hi = lds_tr4(X, pitch, r0 + 16, c0);
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  }
  return r;
}

// The chunk image's fp16 arrays are stored without padding; within a row of
// W halves, the 8-byte piece q (halves 4q .. 4q + 3) of row r sits at piece
// q ^ s(r).  Measured on gfx950 (SQ_LDS_BANK_CONFLICT of probe kernels): an
// 8-byte row read is served 16 lanes at a time over 32 four-byte banks, a
// transposing read 32 lanes at a time over 64 banks.  The row fragment reads
// (16 rows, one piece each) need s distinct modulo 16 over each aligned 16
// rows; the transposing reads (two groups of 4 rows x 4 consecutive pieces)
// need, for rows of 32 pieces, bits 2-4 of s distinct over each aligned 8
// rows and, for rows of 16 pieces (a row pair spans the 64 banks), bits 2-3
// distinct over the 4 rows of one parity among each aligned 8.  s depends on
// the row modulo 16.
template <int W>
__device__ inline int swz_term(int r) {
  if constexpr (W / 4 >= 32)        // 32 pieces: the low four bits with their halves swapped, plus bit 2 as bit 4
    return ((r & 3) << 2) | ((r >> 2) & 3) | (((r >> 2) & 1) << 4);
  else if constexpr (W / 4 == 16)   // 16 pieces: bits 1-2 as bits 2-3, bit 3 as bit 1, bit 0
    return (((r >> 1) & 3) << 2) | (((r >> 3) & 1) << 1) | (r & 1);
  else                              // fewer: the halves-swapped low bits, masked to the row
    return (((r & 3) << 2) | ((r >> 2) & 3)) & (W / 4 - 1);
}
template <int W>
__device__ inline int swz(int r, int c) {
  return (((c >> 2) ^ swz_term<W>(r)) << 2) | (c & 3);
}
// piece q0 (compile-time in the callers) XORed with the lane's term t (below
// the row's piece count, at most 32): the bits above the term's stay an
// immediate offset
template <int W>
__device__ inline int swz_piece(int q0, int t) {
  constexpr int M = W / 4 >= 32 ? 31 : 15;
  return (q0 & ~M) | ((q0 & M) ^ t);
}
// lds_a_perm on a swizzled [*][W] array; row = 16 J + l16 (J compile-time)
template <int W>
__device__ inline f16x8 lds_a_perm_sw(const _Float16* base, int row, int kb, int g,
                                      bool half_only = false) {
  const int t = g ^ swz_term<W>(row);   // kb / 4 is a multiple of 4: g fills bits 0-1
  const _Float16* rp = base + row * W;
  const f16x4 lo = *(const f16x4*)(rp + 4 * swz_piece<W>(kb >> 2, t));
  f16x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  if (half_only) {
    r[4] = r[5] = r[6] = r[7] = (_Float16)0.f;
  } else {
    const f16x4 hi = *(const f16x4*)(rp + 4 * swz_piece<W>((kb + 16) >> 2, t));
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  }
  return r;
}
// lds_tr4 / lds_a_perm_tr on a swizzled [*][W] array; r0 a multiple of 16,
// c0 of 16 (both compile-time in the callers)
template <int W>
__device__ inline f16x4 lds_tr4_sw(const _Float16* X, int r0, int c0) {
  typedef short s16x4_t __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63, s = lane & 15, g = lane >> 4;
  const int rl = 4 * g + (s >> 2);                          // row within the 16-row block
  const int t = (s & 3) ^ swz_term<W>(rl);
  const _Float16* p = X + (r0 + rl) * W + 4 * swz_piece<W>(c0 >> 2, t);
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)p);
  return __builtin_bit_cast(f16x4, v);
}
template <int W>
__device__ inline f16x8 lds_a_perm_tr_sw(const _Float16* X, int r0, int c0, bool half_only = false) {
  const f16x4 lo = lds_tr4_sw<W>(X, r0, c0);
  f16x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  if (half_only) {
    r[4] = r[5] = r[6] = r[7] = (_Float16)0.f;
  } else {
    const f16x4 hi = lds_tr4_sw<W>(X, r0 + 16, c0);
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  }
  return r;
}

template <int BC, int D>
struct Geom {
  static constexpr int NB = BC / 16;               // 16-row blocks of a chunk
  static constexpr int NPAIR = NB * (NB + 1) / 2;  // lower block pairs
  static constexpr int NOFF = NB * (NB - 1) / 2;   // strictly lower block pairs
  static constexpr int NCB = D / 16;               // 16-column blocks of a head dim
  static constexpr int DH = 64;                    // channels per pass of the A/P phase
  static constexpr int NHALF = D / DH;             // passes
  static constexpr int NRG = NT / DH;              // row groups of the element mapping
  static constexpr int RPT = BC / NRG;             // rows per thread in the element mapping
  static constexpr int PH = DH + 8;                // pitch (halves) of [row][DH] hi/lo arrays
  static constexpr int PB = BC + 8;                // pitch (halves) of the chunk pass's [*][BC] fp16 LDS arrays
  static constexpr int PF = BC + 1;                // pitch (floats) of [BC][BC] fp32 arrays
  static_assert(RPT >= 1 && BC % 16 == 0 && D % DH == 0, "geometry");
};

// The chunk images (layouts and sizes in common.h).  VT is the element type
// of V (uint16_t bf16 bits or float); the stored image always reserves fp32
// space for V, and an image with VT = uint16_t is a prefix of it.
template <int BC, int D>
struct FwdHead {   // everything but V: what a forward chunk step keeps in LDS
  _Float16 Qt[BC][D];     // fp16 arrays: rows swizzled (swz), no padding
  _Float16 Kn[BC][D];
  _Float16 KhT[D][BC];
  _Float16 L[BC][BC];
  _Float16 P[BC][BC];
  _Float16 Td[BC][24];
  float gc[D];
  float beta[BC];
  int orow[BC];
};
template <int BC, int D, typename VT>
struct FwdImage : FwdHead<BC, D> {
  VT V[BC][D];   // in 16x16 accumulator-order tiles (state_tile), not row-major
};
static_assert(sizeof(FwdImage<64, 128, float>) == fwd_image_bytes(64, 128), "image layout");
static_assert(sizeof(FwdImage<16, 64, uint16_t>) == fwd_image_used(16, 64, 2), "image layout");
static_assert(sizeof(FwdHead<64, 128>) == fwd_image_head_bytes(64, 128), "image layout");

// One global_load_lds_dwordx4 (the data goes straight to LDS, no registers):
// lane l's 16 bytes at gp go to LDS bytes m + 16 l (m wave-uniform, an LDS
// byte address).  It is issued from inline assembly so that the compiler does
// not see it and places no wait of its own for it before later LDS reads (for
// reads whose memory operands it knows, e.g. the transposing reads, it would
// wait for every copy in flight, however disjoint the addresses); the
// caller's s_waitcnt vmcnt(0) and barrier complete it.  M0 holds the LDS base,
// written in the same statement, one wait state before the load that reads
// it; M0 is a reserved register, which a clobber list cannot protect, so the
// kernels that issue these loads keep nothing else in it (they use no LDS-DMA
// builtin and no indirectly indexed registers, the compiler's uses of M0).
__device__ inline void lds_load16_untracked(const void* gp, unsigned m) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gp), "s"(m)
               : "memory");
}
// The same load with a wave-uniform 64-bit base in SGPRs and a 32-bit
// per-lane byte offset (address = sbase + voff): a copy whose lanes keep one
// offset for all its pieces holds no per-piece 64-bit addresses in registers.
// (Held across a copy, such addresses were spilled to scratch, and the wait
// for a reload waited for the pieces already issued: vector loads complete in
// order.)
__device__ inline void lds_load16_untracked(const void* sbase, unsigned voff, unsigned m) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(m)
               : "memory");
}
// LDS byte address of a shared-memory pointer
__device__ inline unsigned lds_addr(const void* p) {
  return (unsigned)(size_t)(__attribute__((address_space(3))) const char*)p;
}
// Asynchronous copy of `nvec` 16-byte vectors from global memory into LDS by
// such loads: wave w moves the 1 KB pieces w, w + NW, ...; lane l of a piece
// moves its 16 bytes to piece base + 16 l.  Part `part` of NPART of it: each
// wave's pieces split into NPART runs, so that the copy can be issued in
// steps between other work.
template <int NPART = 1>
__device__ inline void lds_copy_async_untracked(void* dst, const unsigned char* src, int nvec,
                                                int part = 0) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const unsigned base = lds_addr(dst), voff = 16u * (unsigned)lane;
  const int per_wave = ((nvec + 63) / 64 + NW - 1) / NW;
  const int j0 = part * per_wave / NPART, j1 = (part + 1) * per_wave / NPART;
  for (int j = j0; j < j1; ++j) {
    const int p = wave + NW * j;
    if (64 * p >= nvec) break;
    if (64 * p + lane < nvec) {
      // the scalar operands made wave-uniform explicitly (at low optimisation
      // levels the compiler does not prove it)
      const size_t sb = (size_t)(src + 1024 * (size_t)p);
      const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)sb);
      const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(sb >> 32));
      lds_load16_untracked((const void*)(((size_t)hi << 32) | lo), voff,
                           __builtin_amdgcn_readfirstlane(base + 1024u * (unsigned)p));
    }
  }
}

// pair index p (0..NPAIR-1) -> block pair (I, J), J <= I, row-major over I
__device__ inline void pair_of(int p, int& I, int& J) {
  I = 0;
  while (p > I) { p -= I + 1; ++I; }
  J = p;
}
// strictly lower pair index of (I, J), J < I
__device__ inline int off_index(int I, int J) { return I * (I - 1) / 2 + J; }

// Shared tables of a chunk: decay references and per-row metadata.
template <int BC, int D>
struct ChunkTables {
  float gref[BC / 16][D];                    // Gam at the first row of each block
  float eref[BC / 16][D];                    // e^gref
  float ecg[BC / 16][D];                     // e^(Gam_C - gref)
  float gc[D];                               // e^Gam_C
  float gcl[D];                              // Gam_C
  float part[Geom<BC, D>::NRG][D];           // per-row-group sums of g
  float dfac[(Geom<BC, D>::NOFF > 0 ? Geom<BC, D>::NOFF : 1)][D];  // e^(gref_I - gref_J)
  float beta[BC];
  int orow[BC];
  int first_bad;   // first row whose in-block decay exceeds kExactDecay (BC: none)
};

// hi/lo operands of the decay-factored products for one 64-channel pass:
//   Lk = K e^(Gam - gref_blk), Lq = Q e^(Gam - gref_blk), Rk = K e^(gref_blk - Gam)
template <int BC, int D>
struct APOps {
  __bf16 kh[BC][Geom<BC, D>::PH], kl[BC][Geom<BC, D>::PH];
  __bf16 qh[BC][Geom<BC, D>::PH], ql[BC][Geom<BC, D>::PH];
  __bf16 rh[BC][Geom<BC, D>::PH], rl[BC][Geom<BC, D>::PH];
};

// Element mapping of the chunk-local pass: thread t owns channels
// t%64 + 64*half (half = 0..NHALF-1) and rows [rg*RPT, (rg+1)*RPT), rg = t/64.
template <int BC, int D>
struct ElemRegs {
  static constexpr int N = Geom<BC, D>::RPT * Geom<BC, D>::NHALF;
  float k[N], q[N], gam[N];   // raw inputs, then Gam
};

// Issues the loads of g, then k, then q for the thread's elements (rows[t] =
// input row of chunk row r0 + t, -1 past the chunk: zeros), in the order the
// chunk pass first needs them (loads return in issue order).  No
// synchronisation.
template <typename TIn, int BC, int D>
__device__ inline void elems_load(const TIn* q, const TIn* k, const float* g, int H, int h,
                                  const int (&rows)[Geom<BC, D>::RPT], ElemRegs<BC, D>& er) {
  using G = Geom<BC, D>;
  const int tid = threadIdx.x;
  const int c0 = tid % G::DH;
  auto off = [&](int hf, int t) {
    const int r = rows[t];
    return ((size_t)(r < 0 ? 0 : r) * H + h) * D + c0 + G::DH * hf;
  };
#pragma unroll
  for (int hf = 0; hf < G::NHALF; ++hf)
#pragma unroll
    for (int t = 0; t < G::RPT; ++t) {
      const float x = g[off(hf, t)];
      er.gam[hf * G::RPT + t] = rows[t] >= 0 ? x : 0.f;
    }
#pragma unroll
  for (int hf = 0; hf < G::NHALF; ++hf)
#pragma unroll
    for (int t = 0; t < G::RPT; ++t) {
      const float x = ld_in(k, off(hf, t));
      er.k[hf * G::RPT + t] = rows[t] >= 0 ? x : 0.f;
    }
#pragma unroll
  for (int hf = 0; hf < G::NHALF; ++hf)
#pragma unroll
    for (int t = 0; t < G::RPT; ++t) {
      const float x = ld_in(q, off(hf, t));
      er.q[hf * G::RPT + t] = rows[t] >= 0 ? x : 0.f;
    }
}

// Gam (cumulative log-decay over the chunk) and the block tables.  Ends
// synchronised.
template <int BC, int D>
__device__ inline void elems_gamma(ChunkTables<BC, D>& tb, ElemRegs<BC, D>& er) {
  using G = Geom<BC, D>;
  const int tid = threadIdx.x;
  const int c0 = tid % G::DH;
  const int rg = tid / G::DH;
  const int r0 = rg * G::RPT;
#pragma unroll
  for (int hf = 0; hf < G::NHALF; ++hf) {
    float run = 0.f;
#pragma unroll
    for (int t = 0; t < G::RPT; ++t) {
      run += er.gam[hf * G::RPT + t];
      er.gam[hf * G::RPT + t] = run;
    }
    tb.part[rg][c0 + G::DH * hf] = run;
  }
  if (tid == 0) tb.first_bad = BC;
  __syncthreads();
#pragma unroll
  for (int hf = 0; hf < G::NHALF; ++hf) {
    const int c = c0 + G::DH * hf;
    float offs = 0.f;
    for (int j = 0; j < rg; ++j) offs += tb.part[j][c];
#pragma unroll
    for (int t = 0; t < G::RPT; ++t) {
      const int n = hf * G::RPT + t;
      er.gam[n] += offs;
      const int i = r0 + t;
      if ((i & 15) == 0) tb.gref[i >> 4][c] = er.gam[n];
      if (i == BC - 1) {
        tb.gc[c] = __expf(er.gam[n]);
        tb.gcl[c] = er.gam[n];
      }
    }
  }
  __syncthreads();
  {  // rows whose decay from their block's first row leaves the factored range
    int bad = BC;
#pragma unroll
    for (int hf = 0; hf < G::NHALF; ++hf)
#pragma unroll
      for (int t = G::RPT - 1; t >= 0; --t) {
        const int i = r0 + t;
        if (tb.gref[i >> 4][c0 + G::DH * hf] - er.gam[hf * G::RPT + t] > kExactDecay) bad = i;
      }
    if (bad < BC) atomicMin(&tb.first_bad, bad);
  }
  if (rg == G::NRG - 1) {
#pragma unroll
    for (int hf = 0; hf < G::NHALF; ++hf) {
      const int c = c0 + G::DH * hf;
      const float gcl = er.gam[hf * G::RPT + G::RPT - 1];  // Gam_C (rows past the chunk add zero)
      for (int b = 0; b < G::NB; ++b) {
        tb.eref[b][c] = __expf(tb.gref[b][c]);
        tb.ecg[b][c] = __expf(gcl - tb.gref[b][c]);
      }
    }
  }
  if (G::NOFF > 0 && tid < D) {
    for (int I = 1; I < G::NB; ++I)
      for (int J = 0; J < I; ++J)
        tb.dfac[off_index(I, J)][tid] = __expf(tb.gref[I][tid] - tb.gref[J][tid]);
  }
  __syncthreads();
}

// Forms the factored operands of pass `hf` (Lk, Lq, Rk around the row's block
// reference) and writes their hi/lo parts to LDS.  No synchronisation.
template <int BC, int D>
__device__ inline void elems_store(int hf, const ElemRegs<BC, D>& er, const ChunkTables<BC, D>& tb,
                                   APOps<BC, D>& ap) {
  using G = Geom<BC, D>;
  const int tid = threadIdx.x;
  const int c0 = tid % G::DH;
  const int r0 = (tid / G::DH) * G::RPT;
#pragma unroll
  for (int t = 0; t < G::RPT; ++t) {
    const int n = hf * G::RPT + t, i = r0 + t;
    const float ref = tb.gref[i >> 4][c0 + G::DH * hf];
    const float f = __expf(er.gam[n] - ref);
    const float fi = __expf(ref - er.gam[n]);
    __bf16 hh, ll;
    split_bf16(er.k[n] * f, hh, ll);
    ap.kh[i][c0] = hh; ap.kl[i][c0] = ll;
    split_bf16(er.q[n] * f, hh, ll);
    ap.qh[i][c0] = hh; ap.ql[i][c0] = ll;
    split_bf16(er.k[n] * fi, hh, ll);
    ap.rh[i][c0] = hh; ap.rl[i][c0] = ll;
  }
}

__device__ inline bf16x8 ld_bf8(const __bf16* p) { return *(const bf16x8*)p; }

// Accumulates one 64-channel pass of A_IJ and P_IJ (block pair (I, J),
// J <= I) on the calling wave; factors taken around gref_J, the channel
// factor between the two references applied once, to the shared operand:
//   A_IJ += Lk_I (Rk_J e^(gref_I - gref_J))^T,  P_IJ += Lq_I (Rk_J e^(...))^T
template <int BC, int D>
__device__ inline void pair_pass(const APOps<BC, D>& ap, const ChunkTables<BC, D>& tb, int hf,
                                 int I, int J, f32x4& accA, f32x4& accP) {
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int g8 = (lane >> 4) * 8;
  const int ri = 16 * I + l16, rj = 16 * J + l16;
  const bool off = I != J;
  const float* df = off ? tb.dfac[off_index(I, J)] + Geom<BC, D>::DH * hf : nullptr;
#pragma unroll
  for (int kb = 0; kb < Geom<BC, D>::DH; kb += 32) {
    const int c0 = kb + g8;
    const bf16x8 kh = ld_bf8(&ap.kh[ri][c0]), kl = ld_bf8(&ap.kl[ri][c0]);
    const bf16x8 qh = ld_bf8(&ap.qh[ri][c0]), ql = ld_bf8(&ap.ql[ri][c0]);
    bf16x8 rh = ld_bf8(&ap.rh[rj][c0]), rl = ld_bf8(&ap.rl[rj][c0]);
    if (off) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        __bf16 h2, l2;
        split_bf16(((float)rh[e] + (float)rl[e]) * df[c0 + e], h2, l2);
        rh[e] = h2; rl[e] = l2;
      }
    }
    accA = mfmab(kh, rh, accA);
    accA = mfmab(kh, rl, accA);
    accA = mfmab(kl, rh, accA);
    accP = mfmab(qh, rh, accP);
    accP = mfmab(qh, rl, accP);
    accP = mfmab(ql, rh, accP);
  }
}

// Full chunk-local A/P phase: loads issued by the caller (elems_load), then
// Gam, the factored operands, and A (strict lower) / P (lower) in fp16 LDS
// arrays [BC][pitch]; blocks above the diagonal are zeroed.  Ends synchronised.
template <int BC, int D>
__device__ inline void chunk_AP(ChunkTables<BC, D>& tb, ElemRegs<BC, D>& er, APOps<BC, D>& ap,
                                _Float16* Aout, int pa, _Float16* Pout, int pp) {
  using G = Geom<BC, D>;
  constexpr int MAXP = (G::NPAIR + NW - 1) / NW;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  elems_gamma<BC, D>(tb, er);
  f32x4 accA[MAXP], accP[MAXP];
#pragma unroll
  for (int m = 0; m < MAXP; ++m) accA[m] = accP[m] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int hf = 0; hf < G::NHALF; ++hf) {
    if (hf > 0) __syncthreads();
    elems_store<BC, D>(hf, er, tb, ap);
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MAXP; ++m) {
      const int p = wave + NW * m;
      if (p < G::NPAIR) {
        int I, J;
        pair_of(p, I, J);
        pair_pass<BC, D>(ap, tb, hf, I, J, accA[m], accP[m]);
      }
    }
  }
  __syncthreads();   // the outputs may take the operands' place
#pragma unroll
  for (int m = 0; m < MAXP; ++m) {
    const int p = wave + NW * m;
    if (p < G::NPAIR) {
      int I, J;
      pair_of(p, I, J);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + (lane >> 4) * 4 + r;
        const int j = 16 * J + (lane & 15);
        Aout[i * pa + j] = (_Float16)((j < i) ? accA[m][r] : 0.f);
        Pout[i * pp + j] = (_Float16)((j <= i) ? accP[m][r] : 0.f);
      }
    }
  }
  for (int e = threadIdx.x; e < BC * BC; e += NT) {
    const int i = e / BC, j = e % BC;
    if ((j >> 4) > (i >> 4)) {
      Aout[i * pa + j] = (_Float16)0.f;
      Pout[i * pp + j] = (_Float16)0.f;
    }
  }
  __syncthreads();
}

// Exact A and P entries for the rows i >= first_bad (called when that row
// exists):
//   A_ij = sum_c k_ic k_jc e^(Gam_ic - Gam_jc)  (j < i),  P_ij = the same with q_i (j <= i),
// every exponential taken of a non-positive difference.  It re-reads q, k and
// g of the chunk's rows (irow: input row per chunk row, -1 past the chunk)
// so that it holds none of the caller's registers; the channels go through
// LDS in passes of CP (stage: 3 BC (CP + 1) floats, not overlapping Aout /
// Pout), Gam as a running sum down each channel; thread t owns the pairs
// e = t + NT m (i = e / BC, j = e % BC).  Overwrites those rows of Aout /
// Pout.  Ends synchronised.
template <typename TIn, int BC, int D>
__device__ inline void chunk_AP_exact(const TIn* q, const TIn* k, const float* g,
                                                         int H, int h, const int* irow,
                                                         int first_bad, float* stage,
                                                         _Float16* Aout, int pa, _Float16* Pout,
                                                         int pp) {
  constexpr int CP = 32, SP = CP + 1;
  constexpr int NPR = (BC * BC + NT - 1) / NT;
  float* kx = stage;
  float* qx = stage + BC * SP;
  float* gx = stage + 2 * BC * SP;
  const int tid = threadIdx.x;
  float a[NPR], p[NPR];
#pragma unroll
  for (int m = 0; m < NPR; ++m) a[m] = p[m] = 0.f;
  for (int cp0 = 0; cp0 < D; cp0 += CP) {
    for (int e = tid; e < BC * CP; e += NT) {
      const int i = e / CP, c = e % CP, r = irow[i];
      const size_t o = ((size_t)(r < 0 ? 0 : r) * H + h) * D + cp0 + c;
      kx[i * SP + c] = r >= 0 ? ld_in(k, o) : 0.f;
      qx[i * SP + c] = r >= 0 ? ld_in(q, o) : 0.f;
      gx[i * SP + c] = r >= 0 ? g[o] : 0.f;
    }
    __syncthreads();
    if (tid < CP) {   // Gam: running sum down the rows of channel cp0 + tid
      float run = 0.f;
      for (int i = 0; i < BC; ++i) {
        run += gx[i * SP + tid];
        gx[i * SP + tid] = run;
      }
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NPR; ++m) {
      const int e = tid + NT * m, i = e / BC, j = e % BC;
      if (e < BC * BC && i >= first_bad && j <= i) {
        float sa = 0.f, sp = 0.f;
#pragma unroll 2
        for (int c = 0; c < CP; ++c) {
          const float t = kx[j * SP + c] * __expf(gx[i * SP + c] - gx[j * SP + c]);
          sa = __builtin_fmaf(kx[i * SP + c], t, sa);
          sp = __builtin_fmaf(qx[i * SP + c], t, sp);
        }
        a[m] += sa;
        p[m] += sp;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int m = 0; m < NPR; ++m) {
    const int e = tid + NT * m, i = e / BC, j = e % BC;
    if (e < BC * BC && i >= first_bad && j <= i) {
      Aout[i * pa + j] = (_Float16)(j < i ? a[m] : 0.f);
      Pout[i * pp + j] = (_Float16)p[m];
    }
  }
  __syncthreads();
}

}  // namespace kda
