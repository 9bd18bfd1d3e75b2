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
// k_prep: one block per (chunk, head) over every chunk of every round, used by
// the reverse pass to recompute everything of a chunk that does not depend on
// the state (Gam, A, P, T, W, U).  The forward itself runs fused per round
// (kda_fwd2.hip).
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

// instantiations launched by the reverse pass (kda_bwd.hip)
template __global__ void k_prep<uint16_t, 64, 128>(FwdArgs);
template __global__ void k_prep<uint16_t, 64, 64>(FwdArgs);
template __global__ void k_prep<uint16_t, 16, 128>(FwdArgs);
template __global__ void k_prep<uint16_t, 16, 64>(FwdArgs);
template __global__ void k_prep<float, 64, 128>(FwdArgs);
template __global__ void k_prep<float, 64, 64>(FwdArgs);
template __global__ void k_prep<float, 16, 128>(FwdArgs);
template __global__ void k_prep<float, 16, 64>(FwdArgs);

}  // namespace kda
