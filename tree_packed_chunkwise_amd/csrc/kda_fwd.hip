// kda_fwd.hip -- forward kernels of tree-packed chunkwise KDA (gfx950).
//
// Chunk algebra (gated delta rule, per head; the recurrence itself is the
// reading fixed for the KDA layers that the HARTS pages name in Table 1 and
// Figure 1(b)).  For a chunk of C rows with start state h (dk x dv):
//   Gam_i = sum_{s<=i} g_s                       per key channel
//   A_ij  = sum_c k_ic k_jc e^(Gam_ic-Gam_jc)    j <  i
//   P_ij  = sum_c q_ic k_jc e^(Gam_ic-Gam_jc)    j <= i
//   T     = (I + diag(beta) A)^-1
//   W     = T diag(beta) (K e^Gam),  U = T diag(beta) V
//   delta = U - W h                              (the delta-rule writes)
//   O     = scale (Q e^Gam h + P delta)
//   h'    = diag(e^Gam_C) h + (K e^(Gam_C - Gam))^T delta
//
// Two launches shapes (HARTS Figure 2(c): all sequences of a round form one
// packed call; a later round starts only from states of earlier rounds):
//   k_prep   one block per (chunk, head) over every chunk of every round:
//            everything that does not depend on the state (Gam, A, P, T, W, U).
//   k_state  one block per (sequence, head, dv slice) of one round: walks the
//            sequence's chunks in order carrying its slice of the state; writes
//            outputs of non-replay rows (Figure C.1(b): replayed rows write no
//            semantic outputs), the start state of every chunk (for the
//            backward), handoff states at chunk ends, and the leaf state.
//
// Decay factors: e^(Gam_i - Gam_j) (j <= i) is split around a reference m
// per 16-row block pair as e^(Gam_i - m) * e^(m - Gam_j), with m = Gam at the
// first row of the column block.  The left factor is <= 1; the right one is
// bounded by the decay of at most 15 consecutive rows.  The reference never
// lies after either row of the pair, so every output row depends only on the
// rows up to it: a chunk shared by two trajectories up to a fork gives the
// same bits before the fork in both, which is what lets the packed tree run
// reproduce the trajectory-expanded run exactly (HARTS abstract: replay keeps
// each trajectory's chunkwise numerical path).
#include "common.h"
#include "gemm.h"
#include "timing.h"

namespace kda {

constexpr int NTHREADS = 256;
constexpr int NWAVES = 4;

template <int BC, int D>
struct PrepSmem {
  float K[BC][D + 1];
  float Q[BC][D + 1];   // q, later K e^Gam, later V
  float G[BC][D + 1];   // Gam
  float A[BC][BC + 1];
  float T[BC][BC + 1];
  float beta[BC];
  int row[BC];
};

// Computes A and P for one 16x16 block pair (I, J), J <= I, on the calling wave.
template <int BC, int D>
__device__ inline void pair_AP(PrepSmem<BC, D>& s, int I, int J, float* Pout) {
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int kq = (lane >> 4) * 8;
  const int mrow = 16 * J;
  f32x4 accA = {0.f, 0.f, 0.f, 0.f};
  f32x4 accP = {0.f, 0.f, 0.f, 0.f};
  const int ri = 16 * I + l16;  // row of the A / P operand
  const int rj = 16 * J + l16;  // row of the key operand
  for (int kb = 0; kb < D; kb += 32) {
    bf16x8 kh, kl, qh, ql, rh, rl;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = kb + kq + e;
      const float m = s.G[mrow][c];
      const float li = __expf(s.G[ri][c] - m);
      const float lj = __expf(m - s.G[rj][c]);
      __bf16 h, l;
      split_bf16(s.K[ri][c] * li, h, l);
      kh[e] = h; kl[e] = l;
      split_bf16(s.Q[ri][c] * li, h, l);
      qh[e] = h; ql[e] = l;
      split_bf16(s.K[rj][c] * lj, h, l);
      rh[e] = h; rl[e] = l;
    }
    accA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, rh, accA, 0, 0, 0);
    accA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, rl, accA, 0, 0, 0);
    accA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, rh, accA, 0, 0, 0);
    accP = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, rh, accP, 0, 0, 0);
    accP = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, rl, accP, 0, 0, 0);
    accP = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql, rh, accP, 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 16 * I + (lane >> 4) * 4 + r;
    const int j = 16 * J + l16;
    s.A[i][j] = (j < i) ? accA[r] : 0.f;
    Pout[i * BC + j] = (j <= i) ? accP[r] : 0.f;
  }
}

template <typename TIn, int BC, int D>
__global__ __launch_bounds__(NTHREADS) void k_prep(FwdArgs a) {
  __shared__ PrepSmem<BC, D> s;
  const int c = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int H = a.H;
  const int row0 = a.plan.chunk_row0[c];
  const int len = a.plan.chunk_len[c];
  const TIn* q = (const TIn*)a.q;
  const TIn* k = (const TIn*)a.k;
  const TIn* v = (const TIn*)a.v;
  const size_t blk = ((size_t)c * H + h);
  float* Wg = a.ws.W + blk * BC * D;
  float* Ug = a.ws.U + blk * BC * D;
  float* Gg = a.ws.Gam + blk * BC * D;
  float* Pg = a.ws.P + blk * BC * BC;
  float* Tg = a.ws.T + blk * BC * BC;
  float* Ag = a.ws.A + blk * BC * BC;

  if (tid < BC) {
    const int r = tid < len ? a.plan.row_index[row0 + tid] : -1;
    s.row[tid] = r;
    s.beta[tid] = r >= 0 ? a.beta[(size_t)r * H + h] : 0.f;
  }
  __syncthreads();
  for (int e = tid; e < BC * D; e += NTHREADS) {
    const int i = e / D, ch = e % D;
    const int r = s.row[i];
    float kv = 0.f, qv = 0.f, gv = 0.f;
    if (r >= 0) {
      const size_t off = ((size_t)r * H + h) * D + ch;
      kv = ld_in(k, off);
      qv = ld_in(q, off);
      gv = a.g[off];
    }
    s.K[i][ch] = kv;
    s.Q[i][ch] = qv;
    s.G[i][ch] = gv;
  }
  __syncthreads();
  // inclusive cumulative sum of the log-decay over the chunk's rows
  for (int ch = tid; ch < D; ch += NTHREADS) {
    float acc = 0.f;
    for (int i = 0; i < BC; ++i) {
      acc += s.G[i][ch];
      s.G[i][ch] = acc;
    }
  }
  __syncthreads();
  // A (strict lower) and P (lower) by 16x16 block pairs
  {
    constexpr int NB = BC / 16;
    constexpr int NPAIR = NB * (NB + 1) / 2;
    const int wave = tid >> 6;
    for (int p = wave; p < NPAIR; p += NWAVES) {
      int I = 0, rem = p;
      while (rem > I) { rem -= I + 1; ++I; }
      pair_AP<BC, D>(s, I, rem, Pg);
    }
  }
  __syncthreads();
  // T = (I + diag(beta) A)^-1, one column per thread (forward substitution)
  for (int j = tid; j < BC; j += NTHREADS) {
    for (int i = 0; i < BC; ++i) {
      float acc = (i == j) ? 1.f : 0.f;
      if (i > j) {
        const float bi = s.beta[i];
        for (int m = j; m < i; ++m) acc -= bi * s.A[i][m] * s.T[m][j];
      }
      s.T[i][j] = (i >= j) ? acc : 0.f;
    }
  }
  // K e^Gam replaces q
  for (int e = tid; e < BC * D; e += NTHREADS) {
    const int i = e / D, ch = e % D;
    s.Q[i][ch] = s.K[i][ch] * __expf(s.G[i][ch]);
  }
  __syncthreads();
  auto tri_skip = [](int i0, int, int kb) { return kb > i0 + 15; };
  // W = T diag(beta) (K e^Gam)
  gemm3<BC, D, BC, NWAVES>(
      [&](int i, int j) { return s.T[i][j] * s.beta[j]; },
      [&](int j, int ch) { return s.Q[j][ch]; },
      [&](int i, int ch, float x) { Wg[i * D + ch] = x; }, tri_skip);
  __syncthreads();
  // V replaces K e^Gam
  for (int e = tid; e < BC * D; e += NTHREADS) {
    const int i = e / D, ch = e % D;
    const int r = s.row[i];
    s.Q[i][ch] = r >= 0 ? ld_in(v, ((size_t)r * H + h) * D + ch) : 0.f;
  }
  __syncthreads();
  gemm3<BC, D, BC, NWAVES>(
      [&](int i, int j) { return s.T[i][j] * s.beta[j]; },
      [&](int j, int ch) { return s.Q[j][ch]; },
      [&](int i, int ch, float x) { Ug[i * D + ch] = x; }, tri_skip);
  for (int e = tid; e < BC * D; e += NTHREADS) Gg[e] = s.G[e / D][e % D];
  for (int e = tid; e < BC * BC; e += NTHREADS) {
    const int i = e / BC, j = e % BC;
    const bool low = j < i;
    Tg[e] = s.T[i][j];
    Ag[e] = low ? s.A[i][j] : 0.f;
    if ((j >> 4) > (i >> 4)) Pg[e] = 0.f;  // blocks above the diagonal
  }
}

template <int BC, int D, int DVS>
struct StateSmem {
  float H[D][DVS + 1];
  float Del[BC][DVS + 1];
  float M[BC][D + 1];
  float P[BC][BC + 1];
  float GC[D];
};

template <typename TIn, int BC, int D, int DVS>
__global__ __launch_bounds__(NTHREADS) void k_state(FwdArgs a, int seq_begin) {
  __shared__ StateSmem<BC, D, DVS> s;
  const int seq = seq_begin + blockIdx.x;
  const int h = blockIdx.y;
  const int v0 = blockIdx.z * DVS;
  const int tid = threadIdx.x;
  const int H = a.H;
  const TIn* q = (const TIn*)a.q;
  const TIn* k = (const TIn*)a.k;
  const size_t DD = (size_t)D * D;

  // initial state slice
  {
    const float* src = nullptr;
    if (a.plan.seq_init_kind[seq] == 0) {
      if (a.h0) src = a.h0 + ((size_t)a.plan.seq_init_idx[seq] * H + h) * DD;
    } else {
      src = a.bufs + ((size_t)a.plan.seq_init_idx[seq] * H + h) * DD;
    }
    for (int e = tid; e < D * DVS; e += NTHREADS) {
      const int r = e / DVS, cc = e % DVS;
      s.H[r][cc] = src ? src[(size_t)r * D + v0 + cc] : 0.f;
    }
  }
  const int cbeg = a.plan.seq_chunk_ptr[seq];
  const int cend = a.plan.seq_chunk_ptr[seq + 1];
  for (int c = cbeg; c < cend; ++c) {
    const int row0 = a.plan.chunk_row0[c];
    const int len = a.plan.chunk_len[c];
    const int nrep = a.plan.chunk_nrep[c];
    const size_t blk = (size_t)c * H + h;
    const float* Wg = a.ws.W + blk * BC * D;
    const float* Ug = a.ws.U + blk * BC * D;
    const float* Gg = a.ws.Gam + blk * BC * D;
    const float* Pg = a.ws.P + blk * BC * BC;
    __syncthreads();
    {
      float* dst = a.chunk_h + blk * DD;
      for (int e = tid; e < D * DVS; e += NTHREADS) {
        const int r = e / DVS, cc = e % DVS;
        dst[(size_t)r * D + v0 + cc] = s.H[r][cc];
      }
    }
    for (int e = tid; e < BC * D; e += NTHREADS) s.M[e / D][e % D] = Wg[e];
    for (int e = tid; e < BC * DVS; e += NTHREADS) {
      const int i = e / DVS, cc = e % DVS;
      s.Del[i][cc] = Ug[i * D + v0 + cc];
    }
    __syncthreads();
    // delta = U - W h
    gemm3<BC, DVS, D, NWAVES>(
        [&](int i, int ch) { return s.M[i][ch]; },
        [&](int ch, int cc) { return s.H[ch][cc]; },
        [&](int i, int cc, float x) { s.Del[i][cc] -= x; });
    __syncthreads();
    // Q e^Gam, and P
    for (int e = tid; e < BC * D; e += NTHREADS) {
      const int i = e / D, ch = e % D;
      float qv = 0.f;
      if (i < len) {
        const int r = a.plan.row_index[row0 + i];
        qv = ld_in(q, ((size_t)r * H + h) * D + ch) * __expf(Gg[e]);
      }
      s.M[i][ch] = qv;
    }
    for (int e = tid; e < BC * BC; e += NTHREADS) s.P[e / BC][e % BC] = Pg[e];
    __syncthreads();
    // O = scale (Q e^Gam h + P delta): one product over the concatenated inner dim
    {
      const float sc = a.scale;
      gemm3<BC, DVS, D + BC, NWAVES>(
          [&](int i, int kk) { return kk < D ? s.M[i][kk] : s.P[i][kk - D]; },
          [&](int kk, int cc) { return kk < D ? s.H[kk][cc] : s.Del[kk - D][cc]; },
          [&](int i, int cc, float x) {
            if (i >= nrep && i < len) {
              const int orow = a.plan.out_row[row0 + i];
              a.o[((size_t)orow * H + h) * D + v0 + cc] = sc * x;
            }
          });
    }
    __syncthreads();
    // K e^(Gam_C - Gam) and e^Gam_C
    for (int e = tid; e < BC * D; e += NTHREADS) {
      const int i = e / D, ch = e % D;
      float kv = 0.f;
      if (i < len) {
        const int r = a.plan.row_index[row0 + i];
        kv = ld_in(k, ((size_t)r * H + h) * D + ch) * __expf(Gg[(BC - 1) * D + ch] - Gg[e]);
      }
      s.M[i][ch] = kv;
    }
    for (int ch = tid; ch < D; ch += NTHREADS) s.GC[ch] = __expf(Gg[(BC - 1) * D + ch]);
    __syncthreads();
    // h' = diag(e^Gam_C) h + (K e^(Gam_C-Gam))^T delta
    gemm3<D, DVS, BC, NWAVES>(
        [&](int ch, int j) { return s.M[j][ch]; },
        [&](int j, int cc) { return s.Del[j][cc]; },
        [&](int ch, int cc, float x) { s.H[ch][cc] = s.GC[ch] * s.H[ch][cc] + x; });
    __syncthreads();
    const int save = a.plan.chunk_save[c];
    if (save >= 0) {
      float* dst = a.bufs + ((size_t)save * H + h) * DD;
      for (int e = tid; e < D * DVS; e += NTHREADS) {
        const int r = e / DVS, cc = e % DVS;
        dst[(size_t)r * D + v0 + cc] = s.H[r][cc];
      }
    }
  }
  __syncthreads();
  {
    float* dst = a.h_leaf + ((size_t)a.plan.seq_leaf[seq] * H + h) * DD;
    for (int e = tid; e < D * DVS; e += NTHREADS) {
      const int r = e / DVS, cc = e % DVS;
      dst[(size_t)r * D + v0 + cc] = s.H[r][cc];
    }
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

template <typename TIn, int BC, int D>
hipError_t launch_fwd_t(const FwdArgs& a, int n_chunks, const int* round_ptr_host, int n_rounds,
                        hipStream_t st) {
  constexpr int DVS = (D == 128) ? 32 : 16;
  if (n_chunks > 0) {
    KDA_LAUNCH("kda_chunk_prep", (k_prep<TIn, BC, D>), dim3(n_chunks, a.H), dim3(NTHREADS), st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  for (int r = 0; r < n_rounds; ++r) {
    const int nseq = round_ptr_host[r + 1] - round_ptr_host[r];
    if (nseq == 0) continue;
    KDA_LAUNCH("kda_fwd_state", (k_state<TIn, BC, D, DVS>), dim3(nseq, a.H, D / DVS),
               dim3(NTHREADS), st, a, round_ptr_host[r]);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_fwd(const FwdArgs& a, bool bf16, int BC, int D, int n_chunks,
                      const int* round_ptr_host, int n_rounds, hipStream_t st) {
#define KDA_FWD_CASE(T, BCv, Dv)                                                         \
  if (BC == BCv && D == Dv) return launch_fwd_t<T, BCv, Dv>(a, n_chunks, round_ptr_host, \
                                                           n_rounds, st);
  if (bf16) {
    KDA_FWD_CASE(uint16_t, 64, 128)
    KDA_FWD_CASE(uint16_t, 64, 64)
    KDA_FWD_CASE(uint16_t, 16, 128)
    KDA_FWD_CASE(uint16_t, 16, 64)
  } else {
    KDA_FWD_CASE(float, 64, 128)
    KDA_FWD_CASE(float, 64, 64)
    KDA_FWD_CASE(float, 16, 128)
    KDA_FWD_CASE(float, 16, 64)
  }
#undef KDA_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace kda
