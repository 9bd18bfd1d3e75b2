// kda_prep.hip -- the chunk-parallel pass: the state-independent part of every
// chunk step, for all chunks of all rounds at once (gfx950).
//
// One block per (chunk, head).  This part of the chunk algebra does not
// depend on the recurrent state, so it runs fully parallel ahead of the
// per-round passes and is shared by the forward and the reverse pass.  Per
// chunk (C rows, HARTS Figure 2(c): a chunk of a packed sequence):
//   Gam_i = sum_{s<=i} g_s                                     per key channel
//   A_ij  = sum_c k_ic k_jc e^(Gam_ic - Gam_jc)   (j < i)
//   P_ij  = sum_c q_ic k_jc e^(Gam_ic - Gam_jc)   (j <= i)
//   Td_I  = (I + diag(beta_I) A_II)^-1 for every 16-row diagonal block I
// and the decayed operands q e^Gam, k e^Gam, k e^(Gam_C - Gam).  Everything
// is written as one chunk image (layout in chunk.h): the LDS image of a
// forward chunk step, whose head the reverse chunk step reads as well (its
// transposed operands come from transposing LDS reads), so that the round
// kernels' sequential chain only copies an image and runs the state phase.
// The state-dependent passes solve (I + diag(beta) A) delta = diag(beta) Z
// (and its transpose) block by block with Td; the full inverse is never
// formed.  Two blocks share a compute unit (70 KB of LDS, 128 registers).
// Chunks with rows whose decay leaves the factored range (any g <= 0 is
// accepted) recompute those rows' A and P pair by pair (chunk.h).
#include "chunk.h"
#include "timing.h"

namespace kda {

template <int BC, int D>
struct PrepSmem {
  using G = Geom<BC, D>;
  union {                     // the products' outputs replace their staged operands
    APOps<BC, D> ap;
    struct {
      _Float16 A[BC][G::PB];
      _Float16 P[BC][G::PB];
    } o;
    struct {                  // the exact path stages channels behind the outputs
      _Float16 A[BC][G::PB];
      _Float16 P[BC][G::PB];
      float stage[3 * BC * 33];
    } x;
  } u;
  ChunkTables<BC, D> tb;
  int irow[BC];   // input row of each chunk row (-1 past the chunk)
};

template <typename TIn>
__device__ inline TIn to_in(float x);
template <>
__device__ inline float to_in<float>(float x) { return x; }
template <>
__device__ inline uint16_t to_in<uint16_t>(float x) {  // exact: x holds a bf16 value
  return (uint16_t)(__float_as_uint(x) >> 16);
}

template <typename TIn, int BC, int D>
__global__ __launch_bounds__(NT) void k_chunk_prep(FwdArgs a, int c_begin) {
  using G = Geom<BC, D>;
  using FI = FwdImage<BC, D, TIn>;
  constexpr int NE = G::RPT * G::NHALF;
  __shared__ PrepSmem<BC, D> s;
  const int c = c_begin + blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int H = a.H;
  const size_t blk = (size_t)c * H + h;
  const int row0 = ld_uni(a.plan.chunk_row0, c);
  const int len = ld_uni(a.plan.chunk_len, c);
  const int nrep = ld_uni(a.plan.chunk_nrep, c);
  // the A/P phase's global loads are issued first (v follows that phase);
  // each thread reads the row indices of its own element rows from the plan
  // (no round trip through a shared table)
  const int c0 = tid % G::DH, r0 = (tid / G::DH) * G::RPT;
  int rows[G::RPT];
#pragma unroll
  for (int t = 0; t < G::RPT; ++t) rows[t] = r0 + t < len ? a.plan.row_index[row0 + r0 + t] : -1;
  int trow = -1, torow = -1;  // row table entries (tid < BC)
  if (tid < BC && tid < len) {
    trow = a.plan.row_index[row0 + tid];
    torow = tid >= nrep ? a.plan.out_row[row0 + tid] : -1;
  }
  // beta, then g, k, q (the A/P phase); the row table goes to LDS after the
  // A/P phase, so that no wait for the later loads comes before it
  const float bx = a.beta[(size_t)(trow < 0 ? 0 : trow) * H + h];
  const float tbeta = trow >= 0 ? bx : 0.f;
  ElemRegs<BC, D> er;
  elems_load<TIn, BC, D>((const TIn*)a.q, (const TIn*)a.k, a.g, H, h, rows, er);
  if (tid < BC) s.irow[tid] = trow;
  chunk_AP<BC, D>(s.tb, er, s.u.ap, &s.u.o.A[0][0], G::PB, &s.u.o.P[0][0], G::PB);
  // v, needed only for the image's V, after the A/P phase (whose final
  // barrier completes the row table): its registers stay free during that
  // phase, and reading the rows back keeps their addresses out of it, so
  // that two blocks fit on a compute unit
#pragma unroll
  for (int t = 0; t < G::RPT; ++t) rows[t] = s.irow[r0 + t];
  float vv[NE];
  {
    const TIn* v = (const TIn*)a.v;
#pragma unroll
    for (int hf = 0; hf < G::NHALF; ++hf)
#pragma unroll
      for (int t = 0; t < G::RPT; ++t) {
        const int r = rows[t];
        const float x = ld_in(v, ((size_t)(r < 0 ? 0 : r) * H + h) * D + c0 + G::DH * hf);
        vv[hf * G::RPT + t] = r >= 0 ? x : 0.f;
      }
  }
  if (tid < BC) {
    s.tb.orow[tid] = torow;
    s.tb.beta[tid] = tbeta;
  }
  FI* F = (FI*)(a.fimg + blk * fwd_image_bytes(BC, D));

  // decayed operands from the element mapping (channel c0 + 64 hf, rows r0..)
#pragma unroll
  for (int hf = 0; hf < G::NHALF; ++hf) {
    const int cc = c0 + G::DH * hf;
    const float gcl = s.tb.gcl[cc];
    _Float16* Fq = &F->Qt[0][0];
    _Float16* Fk = &F->Kn[0][0];
    _Float16 kht[G::RPT];
#pragma unroll
    for (int t = 0; t < G::RPT; ++t) {
      const int n = hf * G::RPT + t, i = r0 + t;
      const float e1 = __expf(er.gam[n]);
      const float e2 = __expf(gcl - er.gam[n]);
      const unsigned o = (unsigned)(i * D + swz<D>(i, cc));   // uniform base + 32-bit offset
      Fq[o] = (_Float16)(er.q[n] * e1);
      Fk[o] = (_Float16)(-er.k[n] * e1);
      kht[t] = (_Float16)(er.k[n] * e2);
    }
    TIn* Vt = &F->V[0][0];   // accumulator-order tiles
    if constexpr (G::RPT % 4 == 0) {   // 4 rows of one column fill one lane's slot of a tile
#pragma unroll
      for (int t = 0; t < G::RPT; t += 4) {
        in4_t<TIn> x;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = to_in<TIn>(vv[hf * G::RPT + t + j]);
        *(in4_t<TIn>*)&Vt[tile_elem<D>(r0 + t, cc)] = x;
      }
    } else {
#pragma unroll
      for (int t = 0; t < G::RPT; ++t) Vt[tile_elem<D>(r0 + t, cc)] = to_in<TIn>(vv[hf * G::RPT + t]);
    }
    if constexpr (G::RPT % 4 == 0) {   // whole 8-byte pieces of the swizzled row
#pragma unroll
      for (int t = 0; t < G::RPT; t += 4) {
        f16x4 x;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = kht[t + j];
        *(f16x4*)&F->KhT[cc][swz<BC>(cc, r0 + t)] = x;
      }
    } else {
#pragma unroll
      for (int t = 0; t < G::RPT; ++t) F->KhT[cc][swz<BC>(cc, r0 + t)] = kht[t];
    }
  }
  if (tid < D) F->gc[tid] = s.tb.gc[tid];
  if (tid < BC) {
    F->beta[tid] = s.tb.beta[tid];
    F->orow[tid] = s.tb.orow[tid];
  }
  // rows past the factored decay range take exact pairs (their registers are
  // free here: the element values have been stored)
  if (s.tb.first_bad < BC)
    chunk_AP_exact<TIn, BC, D>((const TIn*)a.q, (const TIn*)a.k, a.g, H, h, s.irow,
                               s.tb.first_bad, s.u.x.stage, &s.u.o.A[0][0], G::PB,
                               &s.u.o.P[0][0], G::PB);
  // -A and P in 8-byte pieces, into their swizzled places
  for (int e = tid; e < BC * BC / 4; e += NT) {
    const int i = e / (BC / 4), j0 = (e % (BC / 4)) * 4;
    *(f16x4*)&F->L[i][swz<BC>(i, j0)] = -*(const f16x4*)&s.u.o.A[i][j0];
    *(f16x4*)&F->P[i][swz<BC>(i, j0)] = *(const f16x4*)&s.u.o.P[i][j0];
  }
  __syncthreads();  // beta of every row
  // diagonal inverses: one lane per (block, column), forward substitution
  if (tid < 16 * G::NB) {
    const int I = tid >> 4, j = tid & 15, b0 = 16 * I;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const f16x8 a0 = *(const f16x8*)&s.u.o.A[b0 + i][b0];
      const f16x8 a1 = *(const f16x8*)&s.u.o.A[b0 + i][b0 + 8];
      const float bi = s.tb.beta[b0 + i];
      float sum = 0.f;   // sum_{m<i} A_im x_m (fp16 A enters the fma directly), then beta_i once
#pragma unroll
      for (int m = 0; m < i; ++m) sum = __builtin_fmaf((float)(m < 8 ? a0[m] : a1[m - 8]), x[m], sum);
      const float acc = ((i == j) ? 1.f : 0.f) - bi * sum;
      x[i] = (i >= j) ? acc : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) F->Td[b0 + i][j] = (_Float16)x[i];
  }
}

template <typename TIn, int BC, int D>
hipError_t launch_prep_t(const FwdArgs& a, int c_begin, int n_chunks, hipStream_t st) {
  if (n_chunks <= 0) return hipSuccess;
  KDA_LAUNCH("kda_chunk_decay", (k_chunk_prep<TIn, BC, D>), dim3(n_chunks, a.H), dim3(NT), st, a,
             c_begin);
  return hipGetLastError();
}

// chunks c_begin .. c_begin + n_chunks - 1
hipError_t launch_prep(const FwdArgs& a, bool bf16, int BC, int D, int c_begin, int n_chunks,
                       hipStream_t st) {
#define KDA_PREP_CASE(T, BCv, Dv) \
  if (BC == BCv && D == Dv) return launch_prep_t<T, BCv, Dv>(a, c_begin, n_chunks, st);
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
