// attn.hip -- tree-ancestor softmax attention over compact rows, forward and
// backward (gfx950).
//
// HARTS Figure 1(b): full attention reads ancestor keys and values; Figure
// C.1(c): attention over the compact layout with a tree mask.  The query at
// offset i of segment v sees every row of every ancestor segment of v and the
// rows of v at offsets <= i (its root path up to itself), so one compact row
// serves every trajectory through it.
//
//   s_rj = scale q_r . k_j,   o_r = sum_j softmax_j(s_r) v_j,   lse_r = logsumexp_j s_rj
//   backward: delta_r = do_r . o_r,  p_rj = e^(s_rj - lse_r),  dp_rj = do_r . v_j,
//             ds_rj = p_rj (dp_rj - delta_r),  dq_r = scale sum_j ds_rj k_j,
//             dk_j = scale sum_r ds_rj q_r,  dv_j = sum_r p_rj do_r
//
// Tiles of 64 rows; 4 waves per block.  Forward and dq blocks take two
// consecutive query tiles of a segment (128 rows), each wave 32 of them
// against whole key tiles; a dk / dv block takes one key tile, each wave 16
// of its keys against whole query tiles.  Key or query tiles are copied into
// LDS asynchronously, double-buffered.  Scores are formed transposed on bf16 matrix
// cores from the exact bf16 inputs, S^T = K Q^T, so that the accumulator tile
// of probabilities (keys down, queries across) is, split into hi/lo bf16, the
// B operand of O^T = V^T P^T without leaving registers (the k order of the
// 32-deep step is permuted as in chunk.h).  Every product with probabilities
// or score gradients takes them as hi + lo bf16 against exact bf16 inputs:
// about 16 mantissa bits with the fp32 exponent range (normalised
// probabilities over 10^4-10^5 keys sit far below fp16's normal range);
// accumulation is fp32.  Key tiles of
// the dk / dv pass see query tiles of their own segment and of every
// descendant segment; the plan cuts those lists into balanced work items and
// sums the partial results of split tiles in a fixed order.
#include "chunk.h"
#include "timing.h"

namespace kda {

constexpr int AT = 64;    // tile rows
constexpr int ANT = 256;  // threads per attention block

__device__ inline float bf2f(uint16_t x) { return __uint_as_float(((uint32_t)x) << 16); }

// two accumulator tiles (rows 0-15, 16-31 of a 32-deep k step) as hi/lo bf16
// B fragments in register k order (chunk.h)
__device__ inline void pair_hl(const f32x4& t0, const f32x4& t1, bf16x8& hi, bf16x8& lo) {
  const float x[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
  split8(x, hi, lo);
}
// A fragment in register k order from a bf16 [*][pitch] LDS array
__device__ inline bf16x8 lds_a_perm_bf(const uint16_t* base, int pitch, int row, int kb, int g) {
  const uint16_t* p = base + row * pitch + kb + 4 * g;
  const uint2 lo = *(const uint2*)p, hi = *(const uint2*)(p + 16);
  bf16x8 r;
  const __bf16* a = (const __bf16*)&lo;
  const __bf16* b = (const __bf16*)&hi;
#pragma unroll
  for (int e = 0; e < 4; ++e) { r[e] = a[e]; r[4 + e] = b[e]; }
  return r;
}
// A (hi + lo) * B with B's hi/lo parts: A holds exact bf16 values
__device__ inline f32x4 mfma_hl(const bf16x8& a, const bf16x8& bh, const bf16x8& bl, f32x4 c) {
  c = mfmab(a, bh, c);
  return mfmab(a, bl, c);
}
__device__ inline float xmax(float a, float b) { return __builtin_fmaxf(a, b); }

// ---- swizzled tiles ----
// A 64-row tile of a bf16 [N][H][D] tensor in LDS, rows unpadded (2 D bytes);
// the 16-byte chunk c of row r sits at chunk position c ^ swz(r).  The swizzle
// keeps both fragment reads free of bank conflicts whether the LDS serves 128
// or 256 bytes a cycle.  A 16-byte row read, one row per lane of a 16-lane
// group: for d = 128 swz is a bijection on r mod 16 and on each aligned 8 rows
// also a bijection mod 8 (bit 0 is bit 2 ^ bit 3 of r, bits 1-3 are r mod 8).
// The transposing 8-byte read, whose 16 lanes address four consecutive rows x
// two adjacent chunks: swz >> 1 differs between any aligned 4 (and 8) rows.
template <int D>
struct SwTile {
  static constexpr int BYTES = AT * D * 2;
  __device__ static int swz(int r) {
    return D == 128 ? (((r & 7) << 1) | (((r >> 2) ^ (r >> 3)) & 1)) : (((r & 3) << 1) | ((r >> 2) & 1));
  }
  // byte offset of element (r, d)
  __device__ static int off(int r, int d) {
    return r * (2 * D) + ((((d >> 3) ^ swz(r))) << 4) + ((d & 7) << 1);
  }
};

// Asynchronous copy of rows r0 .. r0+n-1 of a bf16 [N][H][D] tensor (head h)
// into a swizzled tile (global_load_lds_dwordx4: straight to LDS).  Each 1 KB
// piece of the tile is one wave instruction: lane l fills chunk position l of
// the piece and so loads the chunk that the swizzle places there; rows past n
// repeat row n-1 (their scores are masked).  The loads are issued outside the
// compiler's wait tracking (chunk.h, lds_load16_untracked): tracked, the
// compiler waited for the next tile's copy before the current tile's first
// transposing LDS read.  Completion: s_waitcnt vmcnt(0) and a barrier, by the
// caller.
template <int D, int NWV>
__device__ inline void tile_dma(unsigned char* dst, const uint16_t* src, int r0, int n, int H, int h) {
  constexpr int LPR = (2 * D) / 16;   // lanes per tile row
  constexpr int RPP = 64 / LPR;       // tile rows per 1 KB piece
  constexpr int NP = AT / RPP;
  // a wave's pieces are NWV RPP rows apart, a multiple of the swizzle's
  // period (16 rows for d = 128, 8 for d = 64): every piece of the wave
  // takes the same swizzled chunk per lane
  static_assert((NWV * RPP) % (D == 128 ? 16 : 8) == 0, "swizzle period");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rl = lane / LPR, pos = lane % LPR;
  const int rb = wave * RPP + rl;
  const int c = pos ^ SwTile<D>::swz(rb);
  const unsigned base = __builtin_amdgcn_readfirstlane(lds_addr(dst) + 1024u * (unsigned)wave);
  if (n == AT) {   // a whole tile: one address, advanced by a fixed row stride
    const uint16_t* s0 = src + ((size_t)(r0 + rb) * H + h) * D + 8 * c;
    const size_t step = (size_t)NWV * RPP * H * D;
#pragma unroll
    for (int j = 0; wave + NWV * j < NP; ++j) lds_load16_untracked(s0 + j * step, base + 1024u * NWV * j);
    return;
  }
#pragma unroll
  for (int j = 0; wave + NWV * j < NP; ++j) {
    const int r = (wave + NWV * j) * RPP + rl;
    const int gr = r0 + (r < n ? r : n - 1);
    lds_load16_untracked(src + ((size_t)gr * H + h) * D + 8 * c, base + 1024u * NWV * j);
  }
}

// 16-byte row piece (8 consecutive k) of a swizzled tile: with r = row0 + l16
// and d = 32 ks + 8 g it is the A fragment of rows row0 .. row0+15, k step ks
template <int D>
__device__ inline bf16x8 tile_row8(const unsigned char* t, int r, int d) {
  return *(const bf16x8*)(t + SwTile<D>::off(r, d));
}
// A fragment of X^T in register k order (chunk.h) from a swizzled tile X:
// rows c0 .. c0+15 of X^T (columns of X), k = rows r0 + {4g..4g+3, 16+4g..16+4g+3}
// of X; two transposing 8-byte reads (chunk.h, lds_tr4)
template <int D>
__device__ inline bf16x8 tile_a_tr(const unsigned char* t, int r0, int c0) {
  typedef short s16x4_t __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63, sl = lane & 15, g = lane >> 4;
  const int d = c0 + 4 * (sl & 3);
  const unsigned char* p0 = t + SwTile<D>::off(r0 + 4 * g + (sl >> 2), d);
  const unsigned char* p1 = t + SwTile<D>::off(r0 + 16 + 4 * g + (sl >> 2), d);
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)p0);
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)p1);
  // join the halves as 16-bit integers and bit-cast the whole vector (a
  // __builtin_bit_cast of a single vector element reads element 0 with this
  // compiler, whatever the index)
  typedef short s16x8_t __attribute__((ext_vector_type(8)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
__device__ inline float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }
// maximum / sum over the four 16-lane rows of a wave, per column (lanes l,
// l^16, l^32, l^48): gfx950 row swaps, no LDS round trip
__device__ inline float max_rows4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = xmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return xmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float sum_rows4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// The key tiles a query-tile pair visits: every ancestor segment's tiles, root
// first, then its own segment's up to the pair's end.  Plan values are
// block-uniform and read by scalar loads (a vector load would share the
// in-order vector counter with the tile copies in flight); the loops look up
// the next tile's place before they wait for the current tile's copy.
struct KeyWalk {
  const int* anc;
  const int* seg_row;
  const int* seg_len;
  int a0, na, seg, own_len;   // own_len: the own segment's rows up to the pair's end
  // first row and length of segment ri of the walk (ri == na: the own segment)
  __device__ void place(int ri, int& row, int& len) const {
    const int sg = ri == na ? seg : ld_uni(anc, a0 + ri);
    row = ld_uni(seg_row, sg);
    len = ri == na ? own_len : ld_uni(seg_len, sg);
  }
};

// Running maximum of the online softmax (log2 units): it moves only when a
// tile's maximum exceeds it by more than this, so probabilities stay below
// 2^8 and most tiles skip the rescale of the accumulators.
constexpr float ATT_MAX_SLACK = 8.f;

// Forward, one block (4 waves) per (pair of consecutive query tiles of a
// segment, head): 128 query rows share every key tile the block copies (the
// block launched for a pair's second tile returns at once).  Wave w owns
// queries 32 w .. +31 of the pair and all 64 keys of every key tile, with its
// own online softmax.  Key tiles (every ancestor segment, then the own
// segment up to the pair's end) are double-buffered by asynchronous copies; a
// wave skips own-segment key tiles wholly past its queries, and a wave with no
// queries (a segment's odd last tile) only helps copy.
template <int D>
__global__ __launch_bounds__(ANT, 2) void k_attn_fwd(AttnArgs a) {
  using T = SwTile<D>;
  constexpr int KD = D / 32, NDB = D / 16;
  constexpr int AQ = 2 * AT;   // query rows of a block
  __shared__ __attribute__((aligned(16))) unsigned char sm[2][2][T::BYTES];  // [stage][K, V]
  const int t = a.qorder[blockIdx.x], h = blockIdx.y, H = a.H;
  const int seg = a.tile_seg[t], qoff = a.tile_off[t];
  if (qoff % AQ != 0) return;    // the second tile of a pair
  const int slen = a.seg_len[seg], srow = a.seg_row[seg];
  const int qlen = min(AQ, slen - qoff);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const bool qany = 32 * wave < qlen;   // the wave has queries
  const float sl2 = a.scale * 1.4426950408889634f;   // scores in log2 units
  bf16x8 qf[2][KD];
  int qpos[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = 32 * wave + 16 * qb + l16;
    const int qrow = srow + qoff + min(qi, qlen - 1);
    qpos[qb] = qoff + qi;
#pragma unroll
    for (int ks = 0; ks < KD; ++ks)
      qf[qb][ks] = *(const bf16x8*)(a.q + ((size_t)qrow * H + h) * D + 32 * ks + 8 * g);
  }
  f32x4 ot[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) ot[db][0] = ot[db][1] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  const int a0 = ld_uni(a.anc_ptr, seg);
  const KeyWalk walk{a.anc, a.seg_row, a.seg_len, a0, ld_uni(a.anc_ptr, seg + 1) - a0, seg, qoff + qlen};
  const int na = walk.na;
  auto stage = [&](int st, int r0, int n) {
    tile_dma<D, ANT / 64>(sm[st][0], a.k, r0, n, H, h);
    tile_dma<D, ANT / 64>(sm[st][1], a.v, r0, n, H, h);
  };
  int ri = 0, k0 = 0, st = 0, rrow, rlen;   // the tile in LDS stage st: segment ri of the walk, rows k0..
  walk.place(0, rrow, rlen);
  stage(0, rrow, min(AT, rlen));
  for (;;) {
    const bool own = ri == na;
    const int klen = min(AT, rlen - k0);
    const bool full = !own && klen == AT;   // no masking needed
    int nri = ri, nk0 = k0 + AT, nrow = rrow, nlen = rlen;
    if (nk0 >= rlen) {
      nri = ri + 1;
      nk0 = 0;
      if (nri <= na) walk.place(nri, nrow, nlen);
    }
    const bool more = nri <= na;
    __builtin_amdgcn_s_waitcnt(0);  // this tile has landed ...
    __syncthreads();                // ... for every wave; the other stage is free
    if (more) stage(st ^ 1, nrow + nk0, min(AT, nlen - nk0));
    if (qany && !(own && k0 > qoff + 32 * wave + 31)) {
      const unsigned char* Kt = sm[st][0];
      const unsigned char* Vt = sm[st][1];
      f32x4 sc[4][2];   // S^T tiles [key block][query block], raw scores
#pragma unroll
      for (int k2 = 0; k2 < 4; k2 += 2) {
        bf16x8 kf[2][KD];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int ks = 0; ks < KD; ++ks) kf[kb][ks] = tile_row8<D>(Kt, 16 * (k2 + kb) + l16, 32 * ks + 8 * g);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KD; ++ks) x = mfmab(kf[kb][ks], qf[qb][ks], x);
            sc[k2 + kb][qb] = x;
          }
      }
      bf16x8 ph[2][2], pl[2][2];   // [32-key step][query block]
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        // the tile's maximum over raw scores (the scale is positive), masked
        // keys at -inf
        float mt = -INFINITY;
        if (full) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) mt = xmax(mt, sc[kb][qb][r]);
        } else {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int j = 16 * kb + 4 * g + r;
              const bool vis = j < klen && (!own || k0 + j <= qpos[qb]);
              const float x = vis ? sc[kb][qb][r] : -INFINITY;
              sc[kb][qb][r] = x;
              mt = xmax(mt, x);
            }
        }
        mt = max_rows4(mt) * sl2;
        const float mn = mt > m[qb] + ATT_MAX_SLACK ? mt : m[qb];
        if (__builtin_amdgcn_ballot_w64(mn != m[qb])) {   // some query's reference moved
          const float alpha = m[qb] == -INFINITY ? 0.f : exp2_(m[qb] - mn);
          l[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db) ot[db][qb] *= alpha;
          m[qb] = mn;
        }
        // a query with no visible key yet keeps mn = -inf: its scores are all
        // -inf and any finite reference gives p = 0
        const float mb = mn == -INFINITY ? 0.f : mn;
        float ps = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = exp2_(__builtin_fmaf(sc[kb][qb][r], sl2, -mb));
            sc[kb][qb][r] = p;
            ps += p;
          }
        l[qb] += ps;   // this lane's keys; the 4 lanes of a query are summed at the end
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) pair_hl(sc[2 * k2][qb], sc[2 * k2 + 1][qb], ph[k2][qb], pl[k2][qb]);
      }
      // O^T += V^T P^T, 32 keys per step
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        bf16x8 vf[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) vf[db] = tile_a_tr<D>(Vt, 32 * k2, 16 * db);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) ot[db][qb] = mfma_hl(vf[db], ph[k2][qb], pl[k2][qb], ot[db][qb]);
      }
    }
    if (!more) break;
    ri = nri; k0 = nk0; rrow = nrow; rlen = nlen; st ^= 1;
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = sum_rows4(l[qb]);
    const int qi = 32 * wave + 16 * qb + l16;
    if (qi < qlen) {
      const int qrow = srow + qoff + qi;
      const float inv = 1.f / lt;
      float* dst = a.o + ((size_t)qrow * H + h) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        *(float4*)(dst + 16 * db + 4 * g) =
            make_float4(ot[db][qb][0] * inv, ot[db][qb][1] * inv, ot[db][qb][2] * inv, ot[db][qb][3] * inv);
      if (g == 0) a.lse[(size_t)qrow * H + h] = (m[qb] + __log2f(lt)) * 0.6931471805599453f;
    }
  }
}

// delta_r = dO_r . o_r, one 16-lane row group per (row, head)
template <int D>
__global__ __launch_bounds__(ANT) void k_attn_delta(AttnArgs a, int64_t n_rh) {
  const int64_t rh = ((int64_t)blockIdx.x * ANT + threadIdx.x) / 16;
  const int part = threadIdx.x & 15;
  float x = 0.f;
  if (rh < n_rh) {
#pragma unroll
    for (int e = 0; e < D / 16; ++e) {
      const size_t off = (size_t)rh * D + part * (D / 16) + e;
      x += bf2f(a.dO[off]) * a.oc[off];
    }
  }
  x = row_sum16(x);
  if (rh < n_rh && part == 0) a.delta[rh] = x;
}

// dq, one block (4 waves) per (pair of consecutive query tiles of a segment,
// head), over the same key tiles as the forward (the block of a pair's second
// tile returns at once).  Wave w owns queries 32 w .. +31 of the pair and
// takes each key tile in two 32-key halves:
//   S^T = K Q^T, dP^T = V dO^T (bf16 matrix cores, exact inputs),
//   P^T = 2^(S^T scale log2e - lse log2e), dS^T = P^T (dP^T - delta),
//   dQ^T += K^T dS^T (K^T from the tile by transposing reads, dS^T hi/lo),
// skipping, as the forward, own-segment key tiles wholly past its queries.
template <int D>
__global__ __launch_bounds__(ANT, 2) void k_attn_dq(AttnArgs a) {
  using T = SwTile<D>;
  constexpr int KD = D / 32, NDB = D / 16;
  constexpr int AQ = 2 * AT;   // query rows of a block
  __shared__ __attribute__((aligned(16))) unsigned char sm[2][2][T::BYTES];  // [stage][K, V]
  const int t = a.qorder[blockIdx.x], h = blockIdx.y, H = a.H;
  const int seg = a.tile_seg[t], qoff = a.tile_off[t];
  if (qoff % AQ != 0) return;    // the second tile of a pair
  const int slen = a.seg_len[seg], srow = a.seg_row[seg];
  const int qlen = min(AQ, slen - qoff);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const bool qany = 32 * wave < qlen;
  const float sl2 = a.scale * 1.4426950408889634f;
  bf16x8 qf[2][KD], df[2][KD];
  int qpos[2];
  float lq[2], dl[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = 32 * wave + 16 * qb + l16;
    const int qrow = srow + qoff + min(qi, qlen - 1);
    qpos[qb] = qoff + qi;
#pragma unroll
    for (int ks = 0; ks < KD; ++ks) {
      qf[qb][ks] = *(const bf16x8*)(a.q + ((size_t)qrow * H + h) * D + 32 * ks + 8 * g);
      df[qb][ks] = *(const bf16x8*)(a.dO + ((size_t)qrow * H + h) * D + 32 * ks + 8 * g);
    }
    lq[qb] = a.lsec[(size_t)qrow * H + h] * 1.4426950408889634f;
    dl[qb] = a.delta[(size_t)qrow * H + h];
  }
  f32x4 acc[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db][0] = acc[db][1] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const int a0 = ld_uni(a.anc_ptr, seg);
  const KeyWalk walk{a.anc, a.seg_row, a.seg_len, a0, ld_uni(a.anc_ptr, seg + 1) - a0, seg, qoff + qlen};
  const int na = walk.na;
  auto stage = [&](int st, int r0, int n) {
    tile_dma<D, ANT / 64>(sm[st][0], a.k, r0, n, H, h);
    tile_dma<D, ANT / 64>(sm[st][1], a.v, r0, n, H, h);
  };
  int ri = 0, k0 = 0, st = 0, rrow, rlen;   // the tile in LDS stage st: segment ri of the walk, rows k0..
  walk.place(0, rrow, rlen);
  stage(0, rrow, min(AT, rlen));
  for (;;) {
    const bool own = ri == na;
    const int klen = min(AT, rlen - k0);
    const bool full = !own && klen == AT;
    int nri = ri, nk0 = k0 + AT, nrow = rrow, nlen = rlen;
    if (nk0 >= rlen) {
      nri = ri + 1;
      nk0 = 0;
      if (nri <= na) walk.place(nri, nrow, nlen);
    }
    const bool more = nri <= na;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (more) stage(st ^ 1, nrow + nk0, min(AT, nlen - nk0));
    if (qany && !(own && k0 > qoff + 32 * wave + 31)) {
      const unsigned char* Kt = sm[st][0];
      const unsigned char* Vt = sm[st][1];
#pragma unroll 1
      for (int kh = 0; kh < 2; ++kh) {   // keys 32 kh .. +31 of the tile
        f32x4 sc[2][2], dp[2][2];
        {
          bf16x8 kf[2][KD];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int ks = 0; ks < KD; ++ks) kf[kb][ks] = tile_row8<D>(Kt, 32 * kh + 16 * kb + l16, 32 * ks + 8 * g);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
              sc[kb][qb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int ks = 0; ks < KD; ++ks) sc[kb][qb] = mfmab(kf[kb][ks], qf[qb][ks], sc[kb][qb]);
            }
        }
        {
          bf16x8 vf[2][KD];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int ks = 0; ks < KD; ++ks) vf[kb][ks] = tile_row8<D>(Vt, 32 * kh + 16 * kb + l16, 32 * ks + 8 * g);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
              dp[kb][qb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int ks = 0; ks < KD; ++ks) dp[kb][qb] = mfmab(vf[kb][ks], df[qb][ks], dp[kb][qb]);
            }
        }
        bf16x8 bh[2], bl[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float p = exp2_(__builtin_fmaf(sc[kb][qb][r], sl2, -lq[qb]));
              if (!full) {
                const int j = 32 * kh + 16 * kb + 4 * g + r;
                p = j < klen && (!own || k0 + j <= qpos[qb]) ? p : 0.f;
              }
              sc[kb][qb][r] = p * (dp[kb][qb][r] - dl[qb]);   // dS^T
            }
          pair_hl(sc[0][qb], sc[1][qb], bh[qb], bl[qb]);
        }
#pragma unroll
        for (int d0 = 0; d0 < NDB; d0 += 4) {
          bf16x8 kt[4];
#pragma unroll
          for (int db = 0; db < 4; ++db) kt[db] = tile_a_tr<D>(Kt, 32 * kh, 16 * (d0 + db));
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) acc[d0 + db][qb] = mfma_hl(kt[db], bh[qb], bl[qb], acc[d0 + db][qb]);
        }
      }
    }
    if (!more) break;
    ri = nri; k0 = nk0; rrow = nrow; rlen = nlen; st ^= 1;
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = 32 * wave + 16 * qb + l16;
    if (qi < qlen) {
      float* dst = a.dq + ((size_t)(srow + qoff + qi) * H + h) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        *(float4*)(dst + 16 * db + 4 * g) = make_float4(a.scale * acc[db][qb][0], a.scale * acc[db][qb][1],
                                                        a.scale * acc[db][qb][2], a.scale * acc[db][qb][3]);
    }
  }
}

// dk / dv, one block (4 waves) per (work item, head): a key tile and a run of
// the query tiles that see it (its own segment's tiles from the key tile on,
// then every descendant segment's tiles).  Wave w owns keys 16 w .. +15 of the
// key tile; per query tile (double-buffered asynchronous copies of its Q and
// dO rows, and its lse and delta):
//   S = Q K^T, dP = dO V^T (bf16 matrix cores; K and V of the wave's keys in
//   registers), P = 2^(S scale log2e - lse log2e), dS = P (dP - delta),
//   dV^T += dO^T P, dK^T += Q^T dS (dO^T, Q^T by transposing reads; P, dS hi/lo).
template <int D>
__global__ __launch_bounds__(ANT, 2) void k_attn_dkv(AttnArgs a) {
  using T = SwTile<D>;
  constexpr int KD = D / 32, NDB = D / 16;
  __shared__ __attribute__((aligned(16))) unsigned char sm[2][2][T::BYTES];  // [stage][Q, dO]
  __shared__ __attribute__((aligned(16))) float sld[2][2][AT];              // [stage][lse log2e, delta]
  const int item = blockIdx.x, h = blockIdx.y, H = a.H;
  const int t = ld_uni(a.kw_tile, item), q0 = ld_uni(a.kw_q0, item), nq = ld_uni(a.kw_nq, item);
  const int slot = ld_uni(a.kw_slot, item);
  const int seg = ld_uni(a.tile_seg, t), koff = ld_uni(a.tile_off, t);
  const int klen = min(AT, ld_uni(a.seg_len, seg) - koff), krow0 = ld_uni(a.seg_row, seg) + koff;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int kj = 16 * wave + l16;              // this lane's key (column of S)
  const int krow = krow0 + min(kj, klen - 1);
  const float sl2 = a.scale * 1.4426950408889634f;
  bf16x8 kb[KD], vb[KD];
#pragma unroll
  for (int ks = 0; ks < KD; ++ks) {
    kb[ks] = *(const bf16x8*)(a.k + ((size_t)krow * H + h) * D + 32 * ks + 8 * g);
    vb[ks] = *(const bf16x8*)(a.v + ((size_t)krow * H + h) * D + 32 * ks + 8 * g);
  }
  f32x4 dkt[NDB], dvt[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dkt[db] = dvt[db] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const int e0 = ld_uni(a.kq_ptr, t) + q0;
  // query tile i of the item: its segment's offset, its length, whether it is
  // in the key tile's own segment, its first row (plan values: scalar loads)
  struct QTile { int qoff, qlen, qrow0; bool own; };
  auto qtile = [&](int i) {
    const int u = ld_uni(a.kq, e0 + i);
    const int qseg = ld_uni(a.tile_seg, u), qoff = ld_uni(a.tile_off, u);
    return QTile{qoff, min(AT, ld_uni(a.seg_len, qseg) - qoff), ld_uni(a.seg_row, qseg) + qoff, qseg == seg};
  };
  float rl = 0.f, rd = 0.f;   // raw lse / delta of row tid of the query tile in flight (tid < 64)
  auto stage = [&](int st, const QTile& q) {
    // lse and delta before the tiles: a wait for them is no wait for the tiles
    // (rows past the tile repeat its last row; their scores are masked)
    if (tid < AT) {
      const size_t o = (size_t)(q.qrow0 + min(tid, q.qlen - 1)) * H + h;
      rl = a.lsec[o];
      rd = a.delta[o];
    }
    tile_dma<D, ANT / 64>(sm[st][0], a.q, q.qrow0, q.qlen, H, h);
    tile_dma<D, ANT / 64>(sm[st][1], a.dO, q.qrow0, q.qlen, H, h);
  };
  QTile cur{0, 0, 0, false};
  if (nq > 0) {
    cur = qtile(0);
    stage(0, cur);
  }
  for (int i = 0, st = 0; i < nq; ++i, st ^= 1) {
    const int qoff = cur.qoff, qlen = cur.qlen;
    const bool own = cur.own;
    const bool full = !own && qlen == AT && klen == AT;
    QTile nxt{0, 0, 0, false};
    if (i + 1 < nq) nxt = qtile(i + 1);   // in flight across the wait below
    __builtin_amdgcn_s_waitcnt(0);   // this query tile has landed (tiles and rl / rd)
    if (tid < AT) {
      sld[st][0][tid] = rl * 1.4426950408889634f;
      sld[st][1][tid] = rd;
    }
    __syncthreads();
    if (i + 1 < nq) stage(st ^ 1, nxt);
    cur = nxt;
    const unsigned char* Qt = sm[st][0];
    const unsigned char* Ot = sm[st][1];
    f32x4 sp[4], dp[4];   // S and dP tiles [query block], then P and dS
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      bf16x8 fq[2][KD], fo[2][KD];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int ks = 0; ks < KD; ++ks) {
          fq[b][ks] = tile_row8<D>(Qt, 32 * half + 16 * b + l16, 32 * ks + 8 * g);
          fo[b][ks] = tile_row8<D>(Ot, 32 * half + 16 * b + l16, 32 * ks + 8 * g);
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        f32x4 x = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KD; ++ks) {
          x = mfmab(fq[b][ks], kb[ks], x);
          y = mfmab(fo[b][ks], vb[ks], y);
        }
        sp[2 * half + b] = x;
        dp[2 * half + b] = y;
      }
    }
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      // lse and delta of this lane's four queries 16 qb + 4 g .. +3 (rows of S)
      const float4 lv = *(const float4*)&sld[st][0][16 * qb + 4 * g];
      const float4 dv = *(const float4*)&sld[st][1][16 * qb + 4 * g];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qq = 16 * qb + 4 * g + r;
        float p = exp2_(__builtin_fmaf(sp[qb][r], sl2, -(&lv.x)[r]));
        if (!full) p = qq < qlen && kj < klen && (!own || koff + kj <= qoff + qq) ? p : 0.f;
        sp[qb][r] = p;
        dp[qb][r] = p * (dp[qb][r] - (&dv.x)[r]);
      }
    }
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) {   // 32-deep k steps over the query tile's rows
      bf16x8 ph, pl, dh, dlo;
      pair_hl(sp[2 * kq], sp[2 * kq + 1], ph, pl);
      pair_hl(dp[2 * kq], dp[2 * kq + 1], dh, dlo);
#pragma unroll
      for (int d0 = 0; d0 < NDB; d0 += 4) {
        bf16x8 fo[4], fq[4];
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          fo[db] = tile_a_tr<D>(Ot, 32 * kq, 16 * (d0 + db));
          fq[db] = tile_a_tr<D>(Qt, 32 * kq, 16 * (d0 + db));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          dvt[d0 + db] = mfma_hl(fo[db], ph, pl, dvt[d0 + db]);
          dkt[d0 + db] = mfma_hl(fq[db], dh, dlo, dkt[d0 + db]);
        }
      }
    }
  }
  // lane holds d = 16 db + 4 g + r of key kj
  if (kj < klen) {
    float* dk;
    float* dv;
    if (slot < 0) {
      dk = a.dk + ((size_t)(krow0 + kj) * H + h) * D;
      dv = a.dv + ((size_t)(krow0 + kj) * H + h) * D;
    } else {
      float* base = a.part + ((size_t)slot * H + h) * 2 * AT * D;
      dk = base + (size_t)kj * D;
      dv = base + (size_t)(AT + kj) * D;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      *(float4*)(dk + 16 * db + 4 * g) =
          make_float4(a.scale * dkt[db][0], a.scale * dkt[db][1], a.scale * dkt[db][2], a.scale * dkt[db][3]);
      *(float4*)(dv + 16 * db + 4 * g) = make_float4(dvt[db][0], dvt[db][1], dvt[db][2], dvt[db][3]);
    }
  }
}

// split key tiles: dk, dv = the sum of their partial slots, in slot order
template <int D>
__global__ __launch_bounds__(ANT) void k_attn_dkv_reduce(AttnArgs a) {
  const int i = blockIdx.x, h = blockIdx.y, H = a.H;
  const int t = a.ks_tile[i], slot0 = a.ks_slot0[i], ns = a.ks_n[i];
  const int seg = a.tile_seg[t], koff = a.tile_off[t];
  const int klen = min(AT, a.seg_len[seg] - koff), krow0 = a.seg_row[seg] + koff;
  constexpr int N4 = 2 * AT * D / 4, D4 = D / 4;                // float4s of a slot, of a row
  const float4* src = (const float4*)(a.part + ((size_t)slot0 * H + h) * 2 * AT * D);
  const size_t stride = (size_t)H * N4;                          // float4s from slot to slot
  for (int e = threadIdx.x; e < N4; e += ANT) {
    const int which = e / (AT * D4), j = (e / D4) % AT, d = 4 * (e % D4);
    if (j >= klen) continue;
    float4 acc = src[e];
#pragma unroll 4
    for (int sl = 1; sl < ns; ++sl) {
      const float4 x = src[sl * stride + e];
      acc.x += x.x;
      acc.y += x.y;
      acc.z += x.z;
      acc.w += x.w;
    }
    float* dst = which == 0 ? a.dk : a.dv;
    *(float4*)(dst + ((size_t)(krow0 + j) * H + h) * D + d) = acc;
  }
}

template <int D>
hipError_t launch_attn_fwd_t(const AttnArgs& a, int n_tiles, hipStream_t st) {
  if (n_tiles <= 0) return hipSuccess;
  KDA_LAUNCH("tree_attn_fwd", (k_attn_fwd<D>), dim3(n_tiles, a.H), dim3(ANT), st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_attn_bwd_t(const AttnArgs& a, int64_t n_rows, int n_tiles, int n_items,
                             int n_split, hipStream_t st) {
  hipError_t e;
  if (n_rows > 0) {
    const int64_t n_rh = n_rows * a.H;
    const int nb = (int)((n_rh * 16 + ANT - 1) / ANT);
    KDA_LAUNCH("tree_attn_delta", (k_attn_delta<D>), dim3(nb), dim3(ANT), st, a, n_rh);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (n_tiles > 0) {
    KDA_LAUNCH("tree_attn_dq", (k_attn_dq<D>), dim3(n_tiles, a.H), dim3(ANT), st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (n_items > 0) {
    KDA_LAUNCH("tree_attn_dkv", (k_attn_dkv<D>), dim3(n_items, a.H), dim3(ANT), st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (n_split > 0) {
    KDA_LAUNCH("tree_attn_dkv_reduce", (k_attn_dkv_reduce<D>), dim3(n_split, a.H), dim3(ANT), st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_attn_fwd(const AttnArgs& a, int D, int n_tiles, hipStream_t st) {
  if (D == 128) return launch_attn_fwd_t<128>(a, n_tiles, st);
  if (D == 64) return launch_attn_fwd_t<64>(a, n_tiles, st);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_bwd(const AttnArgs& a, int D, int64_t n_rows, int n_tiles, int n_items,
                           int n_split, hipStream_t st) {
  if (D == 128) return launch_attn_bwd_t<128>(a, n_rows, n_tiles, n_items, n_split, st);
  if (D == 64) return launch_attn_bwd_t<64>(a, n_rows, n_tiles, n_items, n_split, st);
  return hipErrorInvalidValue;
}

}  // namespace kda
