// kda_grad.hip -- chunk-local gradients of every chunk (gfx950).
//
// One block (8 waves) per (chunk, head), after the state-gradient rounds.  With
// h the chunk's start state (saved by the forward), dh' its end-state gradient
// and dy (kda_bwd.hip), and the saved decay products A and Td:
//   Z      = V - (K e^Gam) h,   delta: (I + diag(beta) A) delta = diag(beta) Z
//   dV     = diag(beta) dy = dZ
//   dbeta  = rowsum(dy * (Z - A delta))
//   dQt    = scale dO h^T,   dKt = -dZ h^T,   dKh = delta dh'^T,   deGC = rowsum(h * dh')
//   dP     = scale dO delta^T (lower),   dA = -dZ delta^T (strict lower)
//   decay-weighted:  dqP_ic  = sum_{j<=i} dP_ij k_jc e^(Gam_ic-Gam_jc)
//                    dkP_jc  = sum_{i>=j} dP_ij q_ic e^(Gam_ic-Gam_jc)
//                    dkAr_ic = sum_{j< i} dA_ij k_jc e^(..),  dkAc_jc = sum_{i> j} dA_ij k_ic e^(..)
//   dq = dQt e^Gam + dqP
//   dk = dKt e^Gam + dKh e^(Gam_C-Gam) + dkP + dkAr + dkAc
//   dGam = dQt Qt + dKt Kt - dKh Kh + q dqP - k dkP + k dkAr - k dkAc  (+ the Gam_C terms
//          sum_j dKh_j Kh_j + deGC e^Gam_C on the last row);  dg = reverse cumsum of dGam
// Gradients of replayed rows go to replay slots (added into their compact rows
// afterwards in a fixed order).
//
// Phases: (1) each wave owns a 16-column block of dv: Z, delta, the dbeta and
// deGC partials in registers, dO / -dZ / delta / h staged in LDS as fp16;
// (2) products contracting dv on fp16 matrix cores; (3) the decay-weighted
// products on hi/lo bf16 matrix cores in 32-channel passes, decay split
// around the first row of the column block as in the forward, with the
// per-pair channel factor applied to output columns; (4) the combine and the
// reverse cumulative sum.
#include "chunk.h"
#include "timing.h"

namespace kda {

template <int BC, int D>
struct GradGeom {
  static constexpr int NB = BC / 16;
  static constexpr int NCB = D / 16;
  static constexpr int NQ = D / 32;              // 32-channel passes of the decay phase
  static constexpr int PD = D + 8;               // fp16 [*][D] pitch
  static constexpr int PB = BC + 8;              // fp16 [*][BC] pitch
  static constexpr int PF = BC + 1;              // fp32 [BC][BC] pitch
  static constexpr int PG = D + 1;               // fp32 [BC][D] pitch
  static constexpr int PQ = BC + 8;              // bf16 [32][BC] pitch of the decay operands
  static constexpr int NLOW = NB * (NB + 1) / 2; // lower 16x16 blocks of dP / dA
};

// lower block pair (I, J), J <= I -> I (I + 1) / 2 + J
__device__ inline int low_index(int I, int J) { return I * (I + 1) / 2 + J; }

template <int BC, int D>
struct GradSmem {
  using G = GradGeom<BC, D>;
  union {
    struct {
      _Float16 A[BC][G::PB];     // A (strict lower)
      _Float16 Td[BC][24];       // diagonal-block inverses
      union {
        _Float16 Kn[BC][G::PD];  // -(K e^Gam)          [i][c], until Z is formed
        _Float16 dO[BC][G::PD];  // scale dO            [i][v]
      } x;
      _Float16 nZ[BC][G::PD];    // -diag(beta) dy      [i][v]
      _Float16 dl[BC][G::PD];    // delta               [j][v]
      _Float16 Hs[D][G::PD];     // h, later dh'        [c][v]
    } p;
    struct {
      __bf16 rh[32][G::PQ], rl[32][G::PQ];   // (K e^(gref - Gam))^T    [c][j]
      __bf16 qh[32][G::PQ], ql[32][G::PQ];   // (Q e^(Gam - gref))^T    [c][i]
      __bf16 kh[32][G::PQ], kl[32][G::PQ];   // (K e^(Gam - gref))^T    [c][i]
      float Gam[BC][G::PG];                  // Gam, replaced by dGam tile by tile
    } d;
  } u;
  float dP[BC][G::PF];
  float dA[BC][G::PF];
  float redb[NW][BC];        // dbeta partials per wave
  float redg[NW][D];         // deGC partials per wave
  float csum[G::NB][D];      // sum_j dKh_jc K_jc e^(Gam_C - Gam_jc) partials per row block
  float gref[G::NB][D];      // Gam at the first row of each block
  float dfac[G::NLOW][D];    // e^(gref_I - gref_J), J <= I
  float part[8][D];
  float degc[D];
  float gcl[D];              // Gam_C
  float beta[BC];
  int row[BC];
  int orow[BC];
};

// destination of a row gradient: the output row, or the replay slot
__device__ inline float* grad_dst(const BwdArgs& a, float* base, float* rep, int c, int i,
                                  int nrep, int row0, int h, int width) {
  if (i < nrep) return rep + ((size_t)(a.plan.chunk_rep0[c] + i) * a.H + h) * width;
  return base + ((size_t)a.plan.out_row[row0 + i] * a.H + h) * width;
}

template <typename TIn, int BC, int D>
__global__ __launch_bounds__(NT) void k_bwd_grad(BwdArgs a) {
  using G = GradGeom<BC, D>;
  constexpr int NB = G::NB, NCB = G::NCB;
  constexpr int KD = D / 32;
  constexpr int KB = (BC + 31) / 32;
  constexpr bool HALF = (BC == 16);
  __shared__ GradSmem<BC, D> s;
  const int c = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int H = a.H;
  const size_t blk = (size_t)c * H + h;
  const size_t DD = (size_t)D * D;
  const int row0 = a.plan.chunk_row0[c], len = a.plan.chunk_len[c], nrep = a.plan.chunk_nrep[c];
  const TIn* q = (const TIn*)a.q;
  const TIn* k = (const TIn*)a.k;
  const TIn* v = (const TIn*)a.v;
  const TIn* dO = (const TIn*)a.dO;
  const float sc = a.scale;

  if (tid < BC) {
    const int r = tid < len ? a.plan.row_index[row0 + tid] : -1;
    s.row[tid] = r;
    s.orow[tid] = (tid >= nrep && tid < len) ? a.plan.out_row[row0 + tid] : -1;
    s.beta[tid] = r >= 0 ? a.beta[(size_t)r * H + h] : 0.f;
  }
  {  // saved A and Td
    const _Float16* src = a.prep + blk * prep_halves(BC);
    for (int e = tid; e < BC * BC / 8; e += NT) {
      const int i = e / (BC / 8), j0 = (e % (BC / 8)) * 8;
      *(f16x8*)&s.u.p.A[i][j0] = *(const f16x8*)(src + i * BC + j0);
    }
    for (int e = tid; e < NB * 256 / 8; e += NT) {
      const int o = 8 * e;
      *(f16x8*)&s.u.p.Td[o / 16][o % 16] = *(const f16x8*)(src + 2 * BC * BC + o);
    }
  }
  __syncthreads();

  // ---- Gam of the chunk; element mapping: channel c0 + 64 hf, rows r0 .. r0+RPT-1 ----
  constexpr int DH = 64, NRG = NT / DH, RPT = BC / NRG, NHF = D / DH;
  const int c0 = tid % DH, rg = tid / DH, r0 = rg * RPT;
  float gm[RPT * NHF];
  {
    float kk[RPT * NHF];
#pragma unroll
    for (int hf = 0; hf < NHF; ++hf) {
      float run = 0.f;
#pragma unroll
      for (int t = 0; t < RPT; ++t) {
        const int r = s.row[r0 + t];
        const size_t off = ((size_t)(r < 0 ? 0 : r) * H + h) * D + c0 + DH * hf;
        const float x = a.g[off], y = ld_in(k, off);
        run += r >= 0 ? x : 0.f;
        gm[hf * RPT + t] = run;
        kk[hf * RPT + t] = r >= 0 ? y : 0.f;
      }
      s.part[rg][c0 + DH * hf] = run;
    }
    __syncthreads();
#pragma unroll
    for (int hf = 0; hf < NHF; ++hf) {
      const int cc = c0 + DH * hf;
      float offs = 0.f, tot = 0.f;
#pragma unroll
      for (int j = 0; j < NRG; ++j) {
        const float pj = s.part[j][cc];
        offs += (j < rg) ? pj : 0.f;
        tot += pj;
      }
      if (rg == 0) s.gcl[cc] = tot;
#pragma unroll
      for (int t = 0; t < RPT; ++t) {
        const int n = hf * RPT + t, i = r0 + t;
        gm[n] += offs;
        if ((i & 15) == 0) s.gref[i >> 4][cc] = gm[n];
        s.u.p.x.Kn[i][cc] = (_Float16)(-kk[n] * __expf(gm[n]));
      }
    }
  }
  __syncthreads();

  // ---- phase 1: wave w < NCB owns column block w of dv ----
  const bool vw = wave < NCB;
  const int col = 16 * wave + l16;
  f32x4 z[NB];
  if (vw) {
    f32x4 hC[NCB];
    const float* hsrc = a.chunk_h + blk * DD;
    const float* dhsrc = a.dhc + blk * DD;
#pragma unroll
    for (int C = 0; C < NCB; ++C)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const size_t o = (size_t)(16 * C + 4 * g + r) * D + col;
        hC[C][r] = hsrc[o];
        float x = hC[C][r] * dhsrc[o];
        s.u.p.Hs[16 * C + 4 * g + r][col] = (_Float16)hC[C][r];
        // deGC partial over this wave's 16 columns (lanes of equal g)
        x += __shfl_xor(x, 1);
        x += __shfl_xor(x, 2);
        x += __shfl_xor(x, 4);
        x += __shfl_xor(x, 8);
        if (l16 == 0) s.redg[wave][16 * C + 4 * g + r] = x;
      }
    f16x8 hb[KD];
#pragma unroll
    for (int ks = 0; ks < KD; ++ks) hb[ks] = acc_pair(hC[2 * ks], hC[2 * ks + 1]);
    // Z = V - (K e^Gam) h
#pragma unroll
    for (int J = 0; J < NB; ++J) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rr = s.row[16 * J + 4 * g + r];
        const float x = ld_in(v, ((size_t)(rr < 0 ? 0 : rr) * H + h) * D + col);
        z[J][r] = rr >= 0 ? x : 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < KD; ++ks)
        z[J] = mfma16(lds_a_perm(&s.u.p.x.Kn[0][0], G::PD, 16 * J + l16, 32 * ks, g), hb[ks], z[J]);
    }
  }
  __syncthreads();  // Kn is dead: dO takes its place
  if (vw) {
    // delta by block forward substitution with the diagonal inverses
    f32x4 d[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      f32x4 rr = z[I];
#pragma unroll
      for (int J = 0; J < I; ++J) {
        f16x4 la = *(const f16x4*)&s.u.p.A[16 * I + l16][16 * J + 4 * g];
#pragma unroll
        for (int e = 0; e < 4; ++e) la[e] = -la[e];
        rr = mfma16k16(la, acc4(d[J]), rr);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) rr[r] *= s.beta[16 * I + 4 * g + r];
      d[I] = mfma16k16(*(const f16x4*)&s.u.p.Td[16 * I + l16][4 * g], acc4(rr),
                      (f32x4){0.f, 0.f, 0.f, 0.f});
    }
    f16x8 db[KB];
#pragma unroll
    for (int ks = 0; ks < KB; ++ks) db[ks] = HALF ? acc_half(d[0]) : acc_pair(d[2 * ks], d[2 * ks + 1]);
    // e = Z - A delta;  dbeta partial = sum over the columns of dy * e;  dV = beta dy
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      f32x4 e = z[I];
#pragma unroll
      for (int ks = 0; ks < KB; ++ks)
        if (32 * ks <= 16 * I + 15) {
          f16x8 aa = lds_a_perm(&s.u.p.A[0][0], G::PB, 16 * I + l16, 32 * ks, g, HALF);
#pragma unroll
          for (int x = 0; x < 8; ++x) aa[x] = -aa[x];
          e = mfma16(aa, db[ks], e);
        }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * g + r;
        float dyv = 0.f, dov = 0.f;
        if (i < len) dyv = a.dy[((size_t)(row0 + i) * H + h) * D + col];
        const int orow = s.orow[i];
        if (orow >= 0) dov = ld_in(dO, ((size_t)orow * H + h) * D + col);
        const float b = s.beta[i];
        float x = dyv * e[r];
        x += __shfl_xor(x, 1);
        x += __shfl_xor(x, 2);
        x += __shfl_xor(x, 4);
        x += __shfl_xor(x, 8);
        if (l16 == 0) s.redb[wave][i] = x;
        if (i < len) grad_dst(a, a.dv, a.rep_dv, c, i, nrep, row0, h, D)[col] = b * dyv;
        s.u.p.x.dO[i][col] = (_Float16)(sc * dov);
        s.u.p.nZ[i][col] = (_Float16)(-b * dyv);
        s.u.p.dl[i][col] = (_Float16)d[I][r];
      }
    }
  }
  __syncthreads();
  if (tid < BC && tid < len) {
    float acc = 0.f;
    for (int w = 0; w < NCB; ++w) acc += s.redb[w][tid];
    *grad_dst(a, a.dbeta, a.rep_db, c, tid, nrep, row0, h, 1) = acc;
  }
  if (tid < D) {
    float acc = 0.f;
    for (int w = 0; w < NCB; ++w) acc += s.redg[w][tid];
    s.degc[tid] = acc;
  }

  // ---- phase 2: products contracting dv (fp16 matrix cores) ----
  // [BC][D] tile (I, C) belongs to wave I + NB (C % 2); m = C / 2 indexes its registers
  constexpr int NTW = NCB / 2;
  const bool tw = wave < 2 * NB;
  const int tI = wave % NB, tu = wave / NB;
  f32x4 dQt[NTW], dKt[NTW], dKh[NTW];
  if (tw) {
#pragma unroll
    for (int m = 0; m < NTW; ++m) {
      const int C = 2 * m + tu;
      f32x4 x1 = {0.f, 0.f, 0.f, 0.f}, x2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KD; ++ks) {
        const f16x8 bh = *(const f16x8*)&s.u.p.Hs[16 * C + l16][32 * ks + 8 * g];
        x1 = mfma16(*(const f16x8*)&s.u.p.x.dO[16 * tI + l16][32 * ks + 8 * g], bh, x1);
        x2 = mfma16(*(const f16x8*)&s.u.p.nZ[16 * tI + l16][32 * ks + 8 * g], bh, x2);
      }
      dQt[m] = x1;
      dKt[m] = x2;
    }
  }
  // dP (j <= i) and dA (j < i): lower 16x16 blocks dealt over the waves
  for (int t = wave; t < 2 * G::NLOW; t += NW) {
    const bool isA = t >= G::NLOW;
    int I, J;
    pair_of(isA ? t - G::NLOW : t, I, J);
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KD; ++ks) {
      const f16x8 aa = isA ? *(const f16x8*)&s.u.p.nZ[16 * I + l16][32 * ks + 8 * g]
                           : *(const f16x8*)&s.u.p.x.dO[16 * I + l16][32 * ks + 8 * g];
      x = mfma16(aa, *(const f16x8*)&s.u.p.dl[16 * J + l16][32 * ks + 8 * g], x);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * I + 4 * g + r, j = 16 * J + l16;
      if (isA) s.dA[i][j] = (j < i) ? x[r] : 0.f;
      else s.dP[i][j] = (j <= i) ? x[r] : 0.f;
    }
  }
  for (int e = tid; e < BC * BC; e += NT) {
    const int i = e / BC, j = e % BC;
    if ((j >> 4) > (i >> 4)) s.dP[i][j] = s.dA[i][j] = 0.f;
  }
  __syncthreads();
  {  // dh' replaces h
    const float* dhsrc = a.dhc + blk * DD;
    for (int e = tid; e < D * D / 4; e += NT) {
      const int r = (4 * e) / D, cc = (4 * e) % D;
      const float4 x = *(const float4*)(dhsrc + (size_t)r * D + cc);
      s.u.p.Hs[r][cc] = (_Float16)x.x;
      s.u.p.Hs[r][cc + 1] = (_Float16)x.y;
      s.u.p.Hs[r][cc + 2] = (_Float16)x.z;
      s.u.p.Hs[r][cc + 3] = (_Float16)x.w;
    }
  }
  __syncthreads();
  if (tw) {
#pragma unroll
    for (int m = 0; m < NTW; ++m) {
      const int C = 2 * m + tu;
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KD; ++ks)
        x = mfma16(*(const f16x8*)&s.u.p.dl[16 * tI + l16][32 * ks + 8 * g],
                   *(const f16x8*)&s.u.p.Hs[16 * C + l16][32 * ks + 8 * g], x);
      dKh[m] = x;
    }
  }
  __syncthreads();  // the fp16 operands are dead: the decay phase takes their space

  // ---- phase 3: decay-weighted products (hi/lo bf16), 32 channels per pass ----
#pragma unroll
  for (int hf = 0; hf < NHF; ++hf)
#pragma unroll
    for (int t = 0; t < RPT; ++t) s.u.d.Gam[r0 + t][c0 + DH * hf] = gm[hf * RPT + t];
  if (tid < D)
    for (int I = 0; I < NB; ++I)
      for (int J = 0; J <= I; ++J)
        s.dfac[low_index(I, J)][tid] = __expf(s.gref[I][tid] - s.gref[J][tid]);
  // staging of a pass: channel cq = tid % 32, rows rq0 .. rq0 + RPQ - 1
  constexpr int RPQ = (BC * 32 + NT - 1) / NT;
  const int cq = tid % 32, rq0 = (tid / 32) * RPQ;
  float csum_acc[NTW];
#pragma unroll
  for (int m = 0; m < NTW; ++m) csum_acc[m] = 0.f;
#pragma unroll
  for (int qp = 0; qp < G::NQ; ++qp) {
    __syncthreads();
#pragma unroll
    for (int t = 0; t < RPQ; ++t) {
      const int i = rq0 + t;
      if (i < BC) {
        const int cc = 32 * qp + cq;
        const int r = s.row[i];
        const size_t off = ((size_t)(r < 0 ? 0 : r) * H + h) * D + cc;
        const float kv = r >= 0 ? ld_in(k, off) : 0.f;
        const float qv = r >= 0 ? ld_in(q, off) : 0.f;
        const float gam = s.u.d.Gam[i][cc];
        const float ref = s.gref[i >> 4][cc];
        const float f = __expf(gam - ref), fi = __expf(ref - gam);
        __bf16 hh, ll;
        split_bf16(kv * fi, hh, ll);
        s.u.d.rh[cq][i] = hh; s.u.d.rl[cq][i] = ll;
        split_bf16(qv * f, hh, ll);
        s.u.d.qh[cq][i] = hh; s.u.d.ql[cq][i] = ll;
        split_bf16(kv * f, hh, ll);
        s.u.d.kh[cq][i] = hh; s.u.d.kl[cq][i] = ll;
      }
    }
    __syncthreads();
    if (tw) {
      const int m = qp;               // tile (tI, C = 2 qp + tu)
      const int cl = 16 * tu + l16;   // channel within the pass
      const int ch = 32 * qp + cl;    // channel in the head
      const int B0 = 16 * tI;
      f32x4 aq = {0.f, 0.f, 0.f, 0.f}, ak = {0.f, 0.f, 0.f, 0.f};   // row side: dqP, dkAr
      f32x4 cp = {0.f, 0.f, 0.f, 0.f}, ca = {0.f, 0.f, 0.f, 0.f};   // column side: dkP, dkAc
      // row side: pairs (tI, J), J <= tI, around gref_J; the channel factor
      // e^(gref_tI - gref_J) scales the output column
      for (int J = 0; J <= tI; ++J) {
        bf16x8 ph, pl, ah, al, bh, bl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int jj = 8 * g + e;
          float pv = 0.f, av = 0.f;
          __bf16 h2 = (__bf16)0.f, l2 = (__bf16)0.f;
          if (jj < 16) {
            pv = s.dP[B0 + l16][16 * J + jj];
            av = s.dA[B0 + l16][16 * J + jj];
            h2 = s.u.d.rh[cl][16 * J + jj];
            l2 = s.u.d.rl[cl][16 * J + jj];
          }
          __bf16 x, y;
          split_bf16(pv, x, y); ph[e] = x; pl[e] = y;
          split_bf16(av, x, y); ah[e] = x; al[e] = y;
          bh[e] = h2; bl[e] = l2;
        }
        f32x4 tp = {0.f, 0.f, 0.f, 0.f}, ta = {0.f, 0.f, 0.f, 0.f};
        tp = mfmab(ph, bh, tp); tp = mfmab(ph, bl, tp); tp = mfmab(pl, bh, tp);
        ta = mfmab(ah, bh, ta); ta = mfmab(ah, bl, ta); ta = mfmab(al, bh, ta);
        const float f = s.dfac[low_index(tI, J)][ch];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          aq[r] += f * tp[r];
          ak[r] += f * ta[r];
        }
      }
      // column side: pairs (I, tI), I >= tI, around gref_tI; channel factor e^(gref_I - gref_tI)
      for (int I = tI; I < NB; ++I) {
        bf16x8 ph, pl, ah, al, qh, ql, kh, kl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int ii = 8 * g + e;
          float pv = 0.f, av = 0.f;
          __bf16 q1 = (__bf16)0.f, q2 = (__bf16)0.f, k1 = (__bf16)0.f, k2 = (__bf16)0.f;
          if (ii < 16) {
            pv = s.dP[16 * I + ii][B0 + l16];
            av = s.dA[16 * I + ii][B0 + l16];
            q1 = s.u.d.qh[cl][16 * I + ii]; q2 = s.u.d.ql[cl][16 * I + ii];
            k1 = s.u.d.kh[cl][16 * I + ii]; k2 = s.u.d.kl[cl][16 * I + ii];
          }
          __bf16 x, y;
          split_bf16(pv, x, y); ph[e] = x; pl[e] = y;
          split_bf16(av, x, y); ah[e] = x; al[e] = y;
          qh[e] = q1; ql[e] = q2; kh[e] = k1; kl[e] = k2;
        }
        f32x4 tp = {0.f, 0.f, 0.f, 0.f}, ta = {0.f, 0.f, 0.f, 0.f};
        tp = mfmab(ph, qh, tp); tp = mfmab(ph, ql, tp); tp = mfmab(pl, qh, tp);
        ta = mfmab(ah, kh, ta); ta = mfmab(ah, kl, ta); ta = mfmab(al, kh, ta);
        const float f = s.dfac[low_index(I, tI)][ch];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          cp[r] += f * tp[r];
          ca[r] += f * ta[r];
        }
      }
      // ---- phase 4 for this tile: dq, dk, dGam ----
      const float gC = s.gcl[ch];
      const float ref = s.gref[tI][ch];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = B0 + 4 * g + r;
        const float gam = s.u.d.Gam[i][ch];
        const float lf = __expf(gam - ref), rf = __expf(ref - gam);
        const float e1 = __expf(gam), e2 = __expf(gC - gam);
        const int rr = s.row[i];
        const size_t off = ((size_t)(rr < 0 ? 0 : rr) * H + h) * D + ch;
        const float kv = rr >= 0 ? ld_in(k, off) : 0.f;
        const float qv = rr >= 0 ? ld_in(q, off) : 0.f;
        const float vq = aq[r] * lf, vkr = ak[r] * lf, vkp = cp[r] * rf, vka = ca[r] * rf;
        const float dq = dQt[m][r] * e1 + vq;
        const float dk = dKt[m][r] * e1 + dKh[m][r] * e2 + vkr + vkp + vka;
        const float kh2 = dKh[m][r] * kv * e2;
        const float dG = dQt[m][r] * qv * e1 + dKt[m][r] * kv * e1 - kh2 + qv * vq +
                         kv * (vkr - vkp - vka);
        csum_acc[m] += kh2;
        s.u.d.Gam[i][ch] = dG;   // (i, ch) belongs to this lane alone from here on
        if (i < len) {
          grad_dst(a, a.dq, a.rep_dq, c, i, nrep, row0, h, D)[ch] = dq;
          grad_dst(a, a.dk, a.rep_dk, c, i, nrep, row0, h, D)[ch] = dk;
        }
      }
    }
  }
  if (tw) {
#pragma unroll
    for (int m = 0; m < NTW; ++m) {
      float cs = csum_acc[m];
      cs += __shfl_xor(cs, 16);
      cs += __shfl_xor(cs, 32);
      if (g == 0) s.csum[tI][32 * m + 16 * tu + l16] = cs;
    }
  }
  __syncthreads();
  // dg = reverse cumulative sum of dGam; the Gam_C terms enter at the last row
  if (tid < D) {
    float acc = s.degc[tid] * __expf(s.gcl[tid]);
    for (int I = 0; I < NB; ++I) acc += s.csum[I][tid];
    for (int i = BC - 1; i >= 0; --i) {
      acc += s.u.d.Gam[i][tid];
      if (i < len) grad_dst(a, a.dg, a.rep_dg, c, i, nrep, row0, h, D)[tid] = acc;
    }
  }
}

template <typename TIn, int BC, int D>
hipError_t launch_grad_t(const BwdArgs& a, int n_chunks, hipStream_t st) {
  if (n_chunks <= 0) return hipSuccess;
  KDA_LAUNCH("kda_bwd_chunk_grad", (k_bwd_grad<TIn, BC, D>), dim3(n_chunks, a.H), dim3(NT), st, a);
  return hipGetLastError();
}

hipError_t launch_grad(const BwdArgs& a, bool bf16, int BC, int D, int n_chunks, hipStream_t st) {
#define KDA_GRAD_CASE(T, BCv, Dv) \
  if (BC == BCv && D == Dv) return launch_grad_t<T, BCv, Dv>(a, n_chunks, st);
  if (bf16) {
    KDA_GRAD_CASE(uint16_t, 64, 128)
    KDA_GRAD_CASE(uint16_t, 64, 64)
    KDA_GRAD_CASE(uint16_t, 16, 128)
    KDA_GRAD_CASE(uint16_t, 16, 64)
  } else {
    KDA_GRAD_CASE(float, 64, 128)
    KDA_GRAD_CASE(float, 64, 64)
    KDA_GRAD_CASE(float, 16, 128)
    KDA_GRAD_CASE(float, 16, 64)
  }
#undef KDA_GRAD_CASE
  return hipErrorInvalidValue;
}

}  // namespace kda
