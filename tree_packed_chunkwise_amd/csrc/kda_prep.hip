// kda_prep.hip -- chunk-local decay products of every chunk (gfx950).
//
// One block per (chunk, head) over all chunks of all rounds: this part of
// the chunk algebra does not depend on the recurrent state, so it runs fully
// parallel ahead of the per-round passes and is shared by the forward and the
// reverse pass.  Per chunk (C rows):
//   Gam_i = sum_{s<=i} g_s                                     per key channel
//   A_ij  = sum_c k_ic k_jc e^(Gam_ic - Gam_jc)   (j < i)
//   P_ij  = sum_c q_ic k_jc e^(Gam_ic - Gam_jc)   (j <= i)
//   Td_I  = (I + diag(beta_I) A_II)^-1 for every 16-row diagonal block I
// Stored per (chunk, head), fp16: A [C][C] (blocks above the diagonal zero),
// P [C][C], Td [C/16][16][16].  The state-dependent passes solve
// (I + diag(beta) A) delta = diag(beta) Z (and its transpose) block by block
// with Td, so the full inverse is never formed.
#include "chunk.h"
#include "timing.h"

namespace kda {

template <int BC, int D>
struct PrepSmem {
  using G = Geom<BC, D>;
  APOps<BC, D> ap;
  _Float16 A[BC][G::PB];
  _Float16 P[BC][G::PB];
  ChunkTables<BC, D> tb;
};

template <typename TIn, int BC, int D>
__global__ __launch_bounds__(NT) void k_chunk_prep(FwdArgs a) {
  using G = Geom<BC, D>;
  __shared__ PrepSmem<BC, D> s;
  const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int H = a.H;
  const int row0 = a.plan.chunk_row0[c];
  const int len = a.plan.chunk_len[c];
  if (tid < BC) {
    const int r = tid < len ? a.plan.row_index[row0 + tid] : -1;
    s.tb.row[tid] = r;
    s.tb.beta[tid] = r >= 0 ? a.beta[(size_t)r * H + h] : 0.f;
  }
  __syncthreads();
  ElemRegs<BC, D> er;
  elems_load<TIn, BC, D>((const TIn*)a.q, (const TIn*)a.k, a.g, H, h, s.tb, er);
  chunk_AP<BC, D>(s.tb, er, s.ap, &s.A[0][0], G::PB, &s.P[0][0], G::PB);
  _Float16* out = a.prep + ((size_t)c * H + h) * prep_halves(BC);
  _Float16* Lg = out;
  _Float16* Pg = out + BC * BC;
  _Float16* Tg = out + 2 * BC * BC;
  // A and P, 8 halves per thread per pass
  for (int e = tid; e < BC * BC / 8; e += NT) {
    const int i = e / (BC / 8), j0 = (e % (BC / 8)) * 8;
    *(f16x8*)(Lg + i * BC + j0) = *(const f16x8*)&s.A[i][j0];
    *(f16x8*)(Pg + i * BC + j0) = *(const f16x8*)&s.P[i][j0];
  }
  // diagonal inverses: one lane per (block, column), forward substitution
  if (tid < 16 * G::NB) {
    const int I = tid >> 4, j = tid & 15, b0 = 16 * I;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const f16x8 a0 = *(const f16x8*)&s.A[b0 + i][b0];
      const f16x8 a1 = *(const f16x8*)&s.A[b0 + i][b0 + 8];
      const float bi = s.tb.beta[b0 + i];
      float acc = (i == j) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < i; ++m) acc -= bi * (float)(m < 8 ? a0[m] : a1[m - 8]) * x[m];
      x[i] = (i >= j) ? acc : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) Tg[(I * 16 + i) * 16 + j] = (_Float16)x[i];
  }
}

template <typename TIn, int BC, int D>
hipError_t launch_prep_t(const FwdArgs& a, int n_chunks, hipStream_t st) {
  if (n_chunks <= 0) return hipSuccess;
  KDA_LAUNCH("kda_chunk_decay", (k_chunk_prep<TIn, BC, D>), dim3(n_chunks, a.H), dim3(NT), st, a);
  return hipGetLastError();
}

hipError_t launch_prep(const FwdArgs& a, bool bf16, int BC, int D, int n_chunks, hipStream_t st) {
#define KDA_PREP_CASE(T, BCv, Dv) \
  if (BC == BCv && D == Dv) return launch_prep_t<T, BCv, Dv>(a, n_chunks, st);
  if (bf16) {
    KDA_PREP_CASE(uint16_t, 64, 128)
    KDA_PREP_CASE(uint16_t, 64, 64)
    KDA_PREP_CASE(uint16_t, 16, 128)
    KDA_PREP_CASE(uint16_t, 16, 64)
  } else {
    KDA_PREP_CASE(float, 64, 128)
    KDA_PREP_CASE(float, 64, 64)
    KDA_PREP_CASE(float, 16, 128)
    KDA_PREP_CASE(float, 16, 64)
  }
#undef KDA_PREP_CASE
  return hipErrorInvalidValue;
}

}  // namespace kda
