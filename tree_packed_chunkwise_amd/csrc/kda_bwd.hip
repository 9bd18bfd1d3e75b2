// kda_bwd.hip -- reverse pass of one packed round: the state-gradient
// recurrence (gfx950).
//
// One block per (sequence, head, dv slice) of the round, rounds in reverse
// order; the block walks its sequence's chunks backwards carrying dh, the
// gradient of the state at the current chunk end (it starts from the leaf
// state's gradient).  Per chunk, with A, P and the diagonal-block inverses Td
// saved by the forward (kda_prep.hip):
//   at a handoff chunk end: dh += start gradients of every sequence that
//        started from that state (later rounds, already final); the total is
//        the handoff state's gradient (HARTS abstract: differentiable
//        boundary-state handoff)
//   ddelta = scale P^T dO + (K e^(Gam_C - Gam)) dh          (dO = 0 on replay rows)
//   dy     : (I + diag(beta) A)^T dy = ddelta                (block back substitution)
//   dh     <- diag(e^Gam_C) dh + scale (Q e^Gam)^T dO - (K e^Gam)^T diag(beta) dy
// and writes dy and the chunk-end dh for the chunk-local gradient pass; the
// sequence's start gradient goes to its slot.  dh, ddelta and dy stay in
// registers (MFMA accumulators reused as B operands, see chunk.h).
#include "chunk.h"
#include "timing.h"

namespace kda {

template <int BC, int D>
struct BwdRoundSmem {
  using G = Geom<BC, D>;
  static constexpr int PTD = 24;
  _Float16 KhA[BC][G::PD];   // K e^(Gam_C - Gam)     [j][c]
  _Float16 QtT[D][G::PB];    // scale (Q e^Gam)^T     [c][i]
  _Float16 KnT[D][G::PB];    // -(K e^Gam)^T          [c][j]
  _Float16 PT[BC][G::PB];    // scale P^T             [j][i]
  _Float16 AT[BC][G::PB];    // A^T                   [i][j]
  _Float16 TdT[BC][PTD];     // Td_I^T at rows 16I..  [16I+i][m] = Td_I[m][i]
  float part[G::NRG][D];
  float gc[D];               // e^Gam_C
  float beta[BC];
  int row[BC];
  int orow[BC];
};

template <typename TIn, int BC, int D, int NV>
__global__ __launch_bounds__(NT) void k_bwd_round(BwdArgs a, int seq_begin) {
  using G = Geom<BC, D>;
  static_assert(NV <= NW, "one column block per wave");
  constexpr int KD = D / 32;
  constexpr int KB = (BC + 31) / 32;
  constexpr bool HALF = (BC == 16);
  constexpr int NE = G::RPT * G::NHALF;
  __shared__ BwdRoundSmem<BC, D> s;
  const int seq = seq_begin + blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const bool sw = wave < NV;
  const int col = 16 * (blockIdx.z * NV + wave) + l16;
  const int H = a.H;
  const TIn* q = (const TIn*)a.q;
  const TIn* k = (const TIn*)a.k;
  const TIn* dO = (const TIn*)a.dO;
  const size_t DD = (size_t)D * D;
  const float sc = a.scale;
  const int c0 = tid % G::DH, rg = tid / G::DH, r0 = rg * G::RPT;

  f32x4 dh[G::NCB];
  {
    const float* src = a.dh_leaf ? a.dh_leaf + ((size_t)a.plan.seq_leaf[seq] * H + h) * DD : nullptr;
#pragma unroll
    for (int C = 0; C < G::NCB; ++C)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        dh[C][r] = (src && sw) ? src[(size_t)(16 * C + 4 * g + r) * D + col] : 0.f;
  }
  const int cbeg = a.plan.seq_chunk_ptr[seq];
  const int cend = a.plan.seq_chunk_ptr[seq + 1];
  for (int c = cend - 1; c >= cbeg; --c) {
    const int row0 = a.plan.chunk_row0[c];
    const int len = a.plan.chunk_len[c];
    const int nrep = a.plan.chunk_nrep[c];
    const size_t blk = (size_t)c * H + h;
    __syncthreads();
    if (tid < BC) {
      const int r = tid < len ? a.plan.row_index[row0 + tid] : -1;
      s.row[tid] = r;
      s.orow[tid] = (tid >= nrep && tid < len) ? a.plan.out_row[row0 + tid] : -1;
      s.beta[tid] = r >= 0 ? a.beta[(size_t)r * H + h] : 0.f;
    }
    {  // saved decay products, transposed into LDS
      const _Float16* src = a.prep + blk * prep_halves(BC);
      constexpr int NV8 = (int)(prep_halves(BC) / 8);
      for (int e = tid; e < NV8; e += NT) {
        const f16x8 x = *(const f16x8*)(src + 8 * e);
        const int hoff = 8 * e;
        if (hoff < BC * BC) {
          const int i = hoff / BC, j0 = hoff % BC;
#pragma unroll
          for (int m = 0; m < 8; ++m) s.AT[j0 + m][i] = x[m];
        } else if (hoff < 2 * BC * BC) {
          const int o = hoff - BC * BC, i = o / BC, j0 = o % BC;
#pragma unroll
          for (int m = 0; m < 8; ++m) s.PT[j0 + m][i] = (_Float16)(sc * (float)x[m]);
        } else {
          const int o = hoff - 2 * BC * BC;
          const int I = o / 256, mm = (o % 256) / 16, i0 = o % 16;
#pragma unroll
          for (int e2 = 0; e2 < 8; ++e2) s.TdT[16 * I + i0 + e2][mm] = x[e2];
        }
      }
    }
    __syncthreads();
    float kk[NE], qq[NE], gm[NE];
    {
      int rows[G::RPT];
#pragma unroll
      for (int t = 0; t < G::RPT; ++t) rows[t] = s.row[r0 + t];
#pragma unroll
      for (int hf = 0; hf < G::NHALF; ++hf)
#pragma unroll
        for (int t = 0; t < G::RPT; ++t) {
          const int n = hf * G::RPT + t, r = rows[t];
          const size_t off = ((size_t)(r < 0 ? 0 : r) * H + h) * D + c0 + G::DH * hf;
          const float x1 = ld_in(k, off), x2 = ld_in(q, off), x3 = a.g[off];
          kk[n] = r >= 0 ? x1 : 0.f;
          qq[n] = r >= 0 ? x2 : 0.f;
          gm[n] = r >= 0 ? x3 : 0.f;
        }
    }
    // dO as B fragments over the chunk rows (register k order), zero on replay rows
    f16x8 dob[KB];
#pragma unroll
    for (int ks = 0; ks < KB; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 32 * ks + (e < 4 ? 4 * g + e : 16 + 4 * g + e - 4);
        float x = 0.f;
        if (i < BC) {
          const int orow = s.orow[i];
          const float y = ld_in(dO, ((size_t)(orow < 0 ? 0 : orow) * H + h) * D + (sw ? col : 0));
          x = orow >= 0 ? y : 0.f;
        }
        dob[ks][e] = (_Float16)x;
      }
#pragma unroll
    for (int hf = 0; hf < G::NHALF; ++hf) {
      float run = 0.f;
#pragma unroll
      for (int t = 0; t < G::RPT; ++t) {
        run += gm[hf * G::RPT + t];
        gm[hf * G::RPT + t] = run;
      }
      s.part[rg][c0 + G::DH * hf] = run;
    }
    __syncthreads();
#pragma unroll
    for (int hf = 0; hf < G::NHALF; ++hf) {
      const int cc = c0 + G::DH * hf;
      float offs = 0.f, tot = 0.f;
#pragma unroll
      for (int j = 0; j < G::NRG; ++j) {
        const float pj = s.part[j][cc];
        offs += (j < rg) ? pj : 0.f;
        tot += pj;
      }
      if (rg == 0) s.gc[cc] = __expf(tot);
#pragma unroll
      for (int t = 0; t < G::RPT; ++t) {
        const int n = hf * G::RPT + t, i = r0 + t;
        const float gam = gm[n] + offs;
        const float e1 = __expf(gam);
        const float e2 = __expf(tot - gam);
        s.KhA[i][cc] = (_Float16)(kk[n] * e2);
        s.QtT[cc][i] = (_Float16)(sc * qq[n] * e1);
        s.KnT[cc][i] = (_Float16)(-kk[n] * e1);
      }
    }
    __syncthreads();

    if (sw) {
      const int save = a.plan.chunk_save[c];
      if (save >= 0) {
        const int p0 = a.plan.buf_cons_ptr[save], p1 = a.plan.buf_cons_ptr[save + 1];
        for (int pi = p0; pi < p1; ++pi) {
          const float* src = a.slot + ((size_t)a.plan.buf_cons[pi] * H + h) * DD;
#pragma unroll
          for (int C = 0; C < G::NCB; ++C)
#pragma unroll
            for (int r = 0; r < 4; ++r) dh[C][r] += src[(size_t)(16 * C + 4 * g + r) * D + col];
        }
        if (a.dh_boundary) {
          float* dst = a.dh_boundary + ((size_t)save * H + h) * DD;
#pragma unroll
          for (int C = 0; C < G::NCB; ++C)
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(size_t)(16 * C + 4 * g + r) * D + col] = dh[C][r];
        }
      }
      {
        float* dst = a.dhc + blk * DD;
#pragma unroll
        for (int C = 0; C < G::NCB; ++C)
#pragma unroll
          for (int r = 0; r < 4; ++r) dst[(size_t)(16 * C + 4 * g + r) * D + col] = dh[C][r];
      }
      f16x8 dhb[KD];
#pragma unroll
      for (int ks = 0; ks < KD; ++ks) dhb[ks] = acc_pair(dh[2 * ks], dh[2 * ks + 1]);
      // ddelta = scale P^T dO + (K e^(Gam_C-Gam)) dh
      f32x4 dd[G::NB];
#pragma unroll
      for (int J = 0; J < G::NB; ++J) {
        dd[J] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KB; ++ks)
          if (32 * ks + 31 >= 16 * J)
            dd[J] = mfma16(lds_a_perm(&s.PT[0][0], G::PB, 16 * J + l16, 32 * ks, g, HALF), dob[ks], dd[J]);
#pragma unroll
        for (int ks = 0; ks < KD; ++ks)
          dd[J] = mfma16(lds_a_perm(&s.KhA[0][0], G::PD, 16 * J + l16, 32 * ks, g), dhb[ks], dd[J]);
      }
      // (I + diag(beta) A)^T dy = ddelta, from the last block up:
      // dy_I = Td_I^T (ddelta_I - sum_{J>I} A_JI^T diag(beta_J) dy_J)
      f32x4 w[G::NB];
#pragma unroll
      for (int I = G::NB - 1; I >= 0; --I) {
        f32x4 rr = dd[I];
#pragma unroll
        for (int J = G::NB - 1; J > I; --J) {
          f16x4 la = *(const f16x4*)&s.AT[16 * I + l16][16 * J + 4 * g];
#pragma unroll
          for (int e = 0; e < 4; ++e) la[e] = -la[e];
          rr = mfma16k16(la, acc4(w[J]), rr);
        }
        const f32x4 dy = mfma16k16(*(const f16x4*)&s.TdT[16 * I + l16][4 * g], acc4(rr),
                                   (f32x4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * I + 4 * g + r;
          w[I][r] = dy[r] * s.beta[i];
          if (i < len) a.dy[((size_t)(row0 + i) * H + h) * D + col] = dy[r];
        }
      }
      f16x8 wb[KB];
#pragma unroll
      for (int ks = 0; ks < KB; ++ks) wb[ks] = HALF ? acc_half(w[0]) : acc_pair(w[2 * ks], w[2 * ks + 1]);
      // dh <- diag(e^Gam_C) dh + scale (Q e^Gam)^T dO - (K e^Gam)^T diag(beta) dy
#pragma unroll
      for (int C = 0; C < G::NCB; ++C) {
#pragma unroll
        for (int r = 0; r < 4; ++r) dh[C][r] *= s.gc[16 * C + 4 * g + r];
#pragma unroll
        for (int ks = 0; ks < KB; ++ks) {
          dh[C] = mfma16(lds_a_perm(&s.QtT[0][0], G::PB, 16 * C + l16, 32 * ks, g, HALF), dob[ks], dh[C]);
          dh[C] = mfma16(lds_a_perm(&s.KnT[0][0], G::PB, 16 * C + l16, 32 * ks, g, HALF), wb[ks], dh[C]);
        }
      }
    }
  }
  if (sw) {
    float* dst = a.slot + ((size_t)seq * H + h) * DD;
#pragma unroll
    for (int C = 0; C < G::NCB; ++C)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(size_t)(16 * C + 4 * g + r) * D + col] = dh[C][r];
  }
}

int round_slices(int nseq, int H, int D);

template <typename TIn, int BC, int D, int NV>
hipError_t launch_bround(const BwdArgs& a, int nseq, int seq0, int slices, hipStream_t st) {
  KDA_LAUNCH("kda_bwd_round", (k_bwd_round<TIn, BC, D, NV>), dim3(nseq, a.H, slices), dim3(NT),
             st, a, seq0);
  return hipGetLastError();
}

template <typename TIn, int BC, int D>
hipError_t launch_brounds_t(const BwdArgs& a, const int* round_ptr_host, int n_rounds,
                            hipStream_t st) {
  constexpr int NCB = D / 16;
  for (int r = n_rounds - 1; r >= 0; --r) {
    const int nseq = round_ptr_host[r + 1] - round_ptr_host[r];
    if (nseq == 0) continue;
    const int sl = round_slices(nseq, a.H, D);
    const int nv = NCB / sl;
    hipError_t e = hipErrorInvalidValue;
    if (nv == NCB) e = launch_bround<TIn, BC, D, NCB>(a, nseq, round_ptr_host[r], sl, st);
    else if (nv == 4) e = launch_bround<TIn, BC, D, 4>(a, nseq, round_ptr_host[r], sl, st);
    else if (nv == 2) e = launch_bround<TIn, BC, D, 2>(a, nseq, round_ptr_host[r], sl, st);
    else if (nv == 1) e = launch_bround<TIn, BC, D, 1>(a, nseq, round_ptr_host[r], sl, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_bwd_rounds(const BwdArgs& a, bool bf16, int BC, int D, const int* round_ptr_host,
                             int n_rounds, hipStream_t st) {
#define KDA_BR_CASE(T, BCv, Dv) \
  if (BC == BCv && D == Dv) return launch_brounds_t<T, BCv, Dv>(a, round_ptr_host, n_rounds, st);
  if (bf16) {
    KDA_BR_CASE(uint16_t, 64, 128)
    KDA_BR_CASE(uint16_t, 64, 64)
    KDA_BR_CASE(uint16_t, 16, 128)
    KDA_BR_CASE(uint16_t, 16, 64)
  } else {
    KDA_BR_CASE(float, 64, 128)
    KDA_BR_CASE(float, 64, 64)
    KDA_BR_CASE(float, 16, 128)
    KDA_BR_CASE(float, 16, 64)
  }
#undef KDA_BR_CASE
  return hipErrorInvalidValue;
}

}  // namespace kda
