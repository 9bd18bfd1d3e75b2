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
// Tiles of 64 rows; 4 waves per block, each wave owning 16 query rows (forward,
// dq) or 16 key rows (dk / dv).  Scores are formed transposed on bf16 matrix
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
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    __bf16 x, y;
    split_bf16(t0[r], x, y);
    hi[r] = x; lo[r] = y;
    split_bf16(t1[r], x, y);
    hi[4 + r] = x; lo[4 + r] = y;
  }
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
__device__ inline float xmax(float a, float b) { return a > b ? a : b; }

// 64 rows x D columns of a bf16 [N][H][D] tensor (rows r0 .. r0+n-1, zero past
// n) into an LDS tile [64][D+8] and, when `tr` is given, transposed into
// [D][72] (both bf16, exact).
template <int D>
__device__ inline void stage_rows(const uint16_t* src, int r0, int n, int H, int h,
                                  uint16_t (*dst)[D + 8], uint16_t (*tr)[AT + 8]) {
  for (int e = threadIdx.x; e < AT * D / 8; e += ANT) {
    const int j = e / (D / 8), d0 = (e % (D / 8)) * 8;
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    if (j < n) x = *(const uint4*)(src + ((size_t)(r0 + j) * H + h) * D + d0);
    if (dst) *(uint4*)&dst[j][d0] = x;
    if (tr) {
      const uint16_t* xs = (const uint16_t*)&x;
#pragma unroll
      for (int m = 0; m < 8; ++m) tr[d0 + m][j] = xs[m];
    }
  }
}

template <int D>
struct AttnFwdSmem {
  uint16_t K[AT][D + 8];     // key rows (bf16)
  uint16_t Vt[D][AT + 8];    // values, transposed (bf16)
};

template <int D>
__global__ __launch_bounds__(ANT) void k_attn_fwd(AttnArgs a) {
  constexpr int KD = D / 32, NDB = D / 16;
  __shared__ AttnFwdSmem<D> s;
  const int t = a.qorder[blockIdx.x], h = blockIdx.y, H = a.H;
  const int seg = a.tile_seg[t], qoff = a.tile_off[t];
  const int slen = a.seg_len[seg], srow = a.seg_row[seg];
  const int qlen = min(AT, slen - qoff);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int qi = 16 * wave + l16;              // this lane's query (column of S^T)
  const int qrow = srow + qoff + min(qi, qlen - 1);
  const int qpos = qoff + qi;                  // offset of the query within its segment
  const float sc = a.scale;
  bf16x8 qb[KD];
#pragma unroll
  for (int ks = 0; ks < KD; ++ks) qb[ks] = *(const bf16x8*)(a.q + ((size_t)qrow * H + h) * D + 32 * ks + 8 * g);
  f32x4 ot[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) ot[db] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  const int a0 = a.anc_ptr[seg], na = a.anc_ptr[seg + 1] - a0;
  for (int ri = 0; ri <= na; ++ri) {
    const bool own = ri == na;
    const int ksg = own ? seg : a.anc[a0 + ri];
    const int r0 = a.seg_row[ksg];
    const int rlen = own ? qoff + qlen : a.seg_len[ksg];
    for (int k0 = 0; k0 < rlen; k0 += AT) {
      const int klen = min(AT, rlen - k0);
      __syncthreads();  // the previous tile's readers are done
      stage_rows<D>(a.k, r0 + k0, klen, H, h, s.K, nullptr);
      stage_rows<D>(a.v, r0 + k0, klen, H, h, nullptr, s.Vt);
      __syncthreads();
      f32x4 st[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        st[kb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KD; ++ks)
          st[kb] = mfmab(*(const bf16x8*)&s.K[16 * kb + l16][32 * ks + 8 * g], qb[ks], st[kb]);
      }
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * kb + 4 * g + r;
          const bool vis = j < klen && (!own || k0 + j <= qpos);
          const float x = vis ? st[kb][r] * sc : -INFINITY;
          st[kb][r] = x;
          mt = xmax(mt, x);
        }
      mt = xmax(mt, __shfl_xor(mt, 16));
      mt = xmax(mt, __shfl_xor(mt, 32));
      const float mn = xmax(m, mt);
      const float alpha = mn == -INFINITY ? 1.f : __expf(m - mn);
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = st[kb][r] == -INFINITY ? 0.f : __expf(st[kb][r] - mn);
          st[kb][r] = p;
          ps += p;
        }
      ps += __shfl_xor(ps, 16);
      ps += __shfl_xor(ps, 32);
      l = l * alpha + ps;
      m = mn;
      bf16x8 ph0, pl0, ph1, pl1;
      pair_hl(st[0], st[1], ph0, pl0);
      pair_hl(st[2], st[3], ph1, pl1);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int r = 0; r < 4; ++r) ot[db][r] *= alpha;
        ot[db] = mfma_hl(lds_a_perm_bf(&s.Vt[0][0], AT + 8, 16 * db + l16, 0, g), ph0, pl0, ot[db]);
        ot[db] = mfma_hl(lds_a_perm_bf(&s.Vt[0][0], AT + 8, 16 * db + l16, 32, g), ph1, pl1, ot[db]);
      }
    }
  }
  if (qi < qlen) {
    const float inv = 1.f / l;
    float* dst = a.o + ((size_t)qrow * H + h) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *(float4*)(dst + 16 * db + 4 * g) =
          make_float4(ot[db][0] * inv, ot[db][1] * inv, ot[db][2] * inv, ot[db][3] * inv);
    if (g == 0) a.lse[(size_t)qrow * H + h] = m + __logf(l);
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

template <int D>
struct AttnDqSmem {
  uint16_t K[AT][D + 8];
  uint16_t V[AT][D + 8];
  uint16_t Kt[D][AT + 8];
};

template <int D>
__global__ __launch_bounds__(ANT) void k_attn_dq(AttnArgs a) {
  constexpr int KD = D / 32, NDB = D / 16;
  __shared__ AttnDqSmem<D> s;
  const int t = a.qorder[blockIdx.x], h = blockIdx.y, H = a.H;
  const int seg = a.tile_seg[t], qoff = a.tile_off[t];
  const int slen = a.seg_len[seg], srow = a.seg_row[seg];
  const int qlen = min(AT, slen - qoff);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int qi = 16 * wave + l16;
  const int qrow = srow + qoff + min(qi, qlen - 1);
  const int qpos = qoff + qi;
  const float sc = a.scale;
  bf16x8 qb[KD], dob[KD];
#pragma unroll
  for (int ks = 0; ks < KD; ++ks) {
    qb[ks] = *(const bf16x8*)(a.q + ((size_t)qrow * H + h) * D + 32 * ks + 8 * g);
    dob[ks] = *(const bf16x8*)(a.dO + ((size_t)qrow * H + h) * D + 32 * ks + 8 * g);
  }
  const float lq = a.lsec[(size_t)qrow * H + h], dq_ = a.delta[(size_t)qrow * H + h];
  f32x4 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const int a0 = a.anc_ptr[seg], na = a.anc_ptr[seg + 1] - a0;
  for (int ri = 0; ri <= na; ++ri) {
    const bool own = ri == na;
    const int ksg = own ? seg : a.anc[a0 + ri];
    const int r0 = a.seg_row[ksg];
    const int rlen = own ? qoff + qlen : a.seg_len[ksg];
    for (int k0 = 0; k0 < rlen; k0 += AT) {
      const int klen = min(AT, rlen - k0);
      __syncthreads();
      stage_rows<D>(a.k, r0 + k0, klen, H, h, s.K, s.Kt);
      stage_rows<D>(a.v, r0 + k0, klen, H, h, s.V, nullptr);
      __syncthreads();
      f32x4 ds[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        f32x4 st = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KD; ++ks) {
          st = mfmab(*(const bf16x8*)&s.K[16 * kb + l16][32 * ks + 8 * g], qb[ks], st);
          dp = mfmab(*(const bf16x8*)&s.V[16 * kb + l16][32 * ks + 8 * g], dob[ks], dp);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * kb + 4 * g + r;
          const bool vis = j < klen && (!own || k0 + j <= qpos);
          const float p = vis ? __expf(st[r] * sc - lq) : 0.f;
          ds[kb][r] = p * (dp[r] - dq_);
        }
      }
      bf16x8 bh0, bl0, bh1, bl1;
      pair_hl(ds[0], ds[1], bh0, bl0);
      pair_hl(ds[2], ds[3], bh1, bl1);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        acc[db] = mfma_hl(lds_a_perm_bf(&s.Kt[0][0], AT + 8, 16 * db + l16, 0, g), bh0, bl0, acc[db]);
        acc[db] = mfma_hl(lds_a_perm_bf(&s.Kt[0][0], AT + 8, 16 * db + l16, 32, g), bh1, bl1, acc[db]);
      }
    }
  }
  if (qi < qlen) {
    float* dst = a.dq + ((size_t)qrow * H + h) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *(float4*)(dst + 16 * db + 4 * g) =
          make_float4(sc * acc[db][0], sc * acc[db][1], sc * acc[db][2], sc * acc[db][3]);
  }
}

template <int D>
struct AttnDkvSmem {
  uint16_t Q[AT][D + 8];
  uint16_t dO[AT][D + 8];
  uint16_t Qt[D][AT + 8];
  uint16_t dOt[D][AT + 8];
  float lse[AT];
  float delta[AT];
};

template <int D>
__global__ __launch_bounds__(ANT) void k_attn_dkv(AttnArgs a) {
  constexpr int KD = D / 32, NDB = D / 16;
  __shared__ AttnDkvSmem<D> s;
  const int item = blockIdx.x, h = blockIdx.y, H = a.H;
  const int t = a.kw_tile[item], q0 = a.kw_q0[item], nq = a.kw_nq[item], slot = a.kw_slot[item];
  const int seg = a.tile_seg[t], koff = a.tile_off[t];
  const int klen = min(AT, a.seg_len[seg] - koff), krow0 = a.seg_row[seg] + koff;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int kj = 16 * wave + l16;              // this lane's key (column of S)
  const int krow = krow0 + min(kj, klen - 1);
  const float sc = a.scale;
  bf16x8 kb[KD], vb[KD];
#pragma unroll
  for (int ks = 0; ks < KD; ++ks) {
    kb[ks] = *(const bf16x8*)(a.k + ((size_t)krow * H + h) * D + 32 * ks + 8 * g);
    vb[ks] = *(const bf16x8*)(a.v + ((size_t)krow * H + h) * D + 32 * ks + 8 * g);
  }
  f32x4 dkt[NDB], dvt[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dkt[db] = dvt[db] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const int e0 = a.kq_ptr[t] + q0;
  for (int qi_ = 0; qi_ < nq; ++qi_) {
    const int u = a.kq[e0 + qi_];
    const int qseg = a.tile_seg[u], qoff = a.tile_off[u];
    const int qlen = min(AT, a.seg_len[qseg] - qoff), qrow0 = a.seg_row[qseg] + qoff;
    const bool own = qseg == seg;
    __syncthreads();
    stage_rows<D>(a.q, qrow0, qlen, H, h, s.Q, s.Qt);
    stage_rows<D>(a.dO, qrow0, qlen, H, h, s.dO, s.dOt);
    if (tid < AT) {
      const bool ok = tid < qlen;
      s.lse[tid] = ok ? a.lsec[(size_t)(qrow0 + tid) * H + h] : 0.f;
      s.delta[tid] = ok ? a.delta[(size_t)(qrow0 + tid) * H + h] : 0.f;
    }
    __syncthreads();
    f32x4 p[4], ds[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      f32x4 st = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KD; ++ks) {
        st = mfmab(*(const bf16x8*)&s.Q[16 * qb + l16][32 * ks + 8 * g], kb[ks], st);
        dp = mfmab(*(const bf16x8*)&s.dO[16 * qb + l16][32 * ks + 8 * g], vb[ks], dp);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qq = 16 * qb + 4 * g + r;    // query of this element (row of S)
        const bool vis = qq < qlen && kj < klen && (!own || koff + kj <= qoff + qq);
        const float pr = vis ? __expf(st[r] * sc - s.lse[qq]) : 0.f;
        p[qb][r] = pr;
        ds[qb][r] = pr * (dp[r] - s.delta[qq]);
      }
    }
    bf16x8 ph0, pl0, ph1, pl1, dh0, dl0, dh1, dl1;
    pair_hl(p[0], p[1], ph0, pl0);
    pair_hl(p[2], p[3], ph1, pl1);
    pair_hl(ds[0], ds[1], dh0, dl0);
    pair_hl(ds[2], ds[3], dh1, dl1);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      dvt[db] = mfma_hl(lds_a_perm_bf(&s.dOt[0][0], AT + 8, 16 * db + l16, 0, g), ph0, pl0, dvt[db]);
      dvt[db] = mfma_hl(lds_a_perm_bf(&s.dOt[0][0], AT + 8, 16 * db + l16, 32, g), ph1, pl1, dvt[db]);
      dkt[db] = mfma_hl(lds_a_perm_bf(&s.Qt[0][0], AT + 8, 16 * db + l16, 0, g), dh0, dl0, dkt[db]);
      dkt[db] = mfma_hl(lds_a_perm_bf(&s.Qt[0][0], AT + 8, 16 * db + l16, 32, g), dh1, dl1, dkt[db]);
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
          make_float4(sc * dkt[db][0], sc * dkt[db][1], sc * dkt[db][2], sc * dkt[db][3]);
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
  for (int e = threadIdx.x; e < 2 * AT * D; e += ANT) {
    const int which = e / (AT * D), j = (e / D) % AT, d = e % D;
    if (j >= klen) continue;
    float acc = 0.f;
    for (int sl = 0; sl < ns; ++sl) acc += a.part[((size_t)(slot0 + sl) * H + h) * 2 * AT * D + e];
    float* dst = which == 0 ? a.dk : a.dv;
    dst[((size_t)(krow0 + j) * H + h) * D + d] = acc;
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
