// kda_bwd.hip -- reverse-mode kernels of tree-packed chunkwise KDA (gfx950).
//
// Reverse mode of the chunk algebra of kda_fwd.hip.  Per chunk, with start
// state h, end-state gradient dh' and output gradient dO (zero on replayed
// rows, which write no outputs):
//   ddelta = scale P^T dO + (K e^(Gam_C-Gam)) dh'
//   dy     = T^T ddelta
//   dh     = diag(e^Gam_C) dh' + scale (Q e^Gam)^T dO - (diag(beta) K e^Gam)^T dy
//   dV     = diag(beta) dy
//   dbeta  = rowsum(dy * (V - (K e^Gam) h - A delta))
//   dP     = scale dO delta^T (lower),  dA = -diag(beta) dy delta^T (strict lower)
//   dq, dk, dGam through e^Gam, e^(Gam_C-Gam), A and P; dg = reverse cumsum of dGam.
//
// Launches, in stream order:
//   k_prep (shared with the forward)    recompute Gam, A, P, T, W, U per chunk
//   k_bstate, rounds in reverse          the state-gradient recurrence per
//            (sequence, head, dv slice): injects, at every handoff chunk end, the
//            start gradients of the sequences that started from that state (all
//            from later rounds, so already final), writes dy, the end-state
//            gradient of every chunk, each handoff state's total gradient and
//            each sequence's start gradient
//   k_gdelta, k_ghprod, k_gdhprod, k_gsmall, k_gfinal   per (chunk, head):
//            the chunk-local gradients; replayed rows go to replay slots
//   k_reduce_rep   adds replay-slot gradients into their compact rows
//   k_reduce_dh0   sums the start gradients of the sequences that began at each
//                  root's h0
// Every sum has a fixed order: results are bitwise reproducible.
#include "common.h"
#include "gemm.h"
#include "timing.h"

namespace kda {

constexpr int BT = 256;  // threads per block
constexpr int BW = 4;    // waves per block

template <typename TIn, int BC, int D>
__global__ void k_prep(FwdArgs a);  // kda_fwd.hip
hipError_t launch_bwd_rounds(const BwdArgs& a, bool bf16, int BC, int D, const int* round_ptr_host,
                             int n_rounds, hipStream_t st);  // kda_bwd2.hip

// ---------------------------------------------------------------------------
// state-gradient recurrence
// ---------------------------------------------------------------------------
template <int BC, int D, int DVS>
struct BStateSmem {
  float DH[D][DVS + 1];
  float DO[BC][DVS + 1];
  float DD[BC][DVS + 1];
  float DY[BC][DVS + 1];
  float M[BC][D + 1];
  float P[BC][BC + 1];
  float GC[D];
};

template <typename TIn, int BC, int D, int DVS>
__global__ __launch_bounds__(BT) void k_bstate(BwdArgs a, int seq_begin) {
  __shared__ BStateSmem<BC, D, DVS> s;
  const int seq = seq_begin + blockIdx.x;
  const int h = blockIdx.y;
  const int v0 = blockIdx.z * DVS;
  const int tid = threadIdx.x;
  const int H = a.H;
  const TIn* q = (const TIn*)a.q;
  const TIn* k = (const TIn*)a.k;
  const TIn* dO = (const TIn*)a.dO;
  const size_t DD = (size_t)D * D;
  const float sc = a.scale;

  {
    const float* src = a.dh_leaf ? a.dh_leaf + ((size_t)a.plan.seq_leaf[seq] * H + h) * DD : nullptr;
    for (int e = tid; e < D * DVS; e += BT) {
      const int r = e / DVS, cc = e % DVS;
      s.DH[r][cc] = src ? src[(size_t)r * D + v0 + cc] : 0.f;
    }
  }
  const int cbeg = a.plan.seq_chunk_ptr[seq];
  const int cend = a.plan.seq_chunk_ptr[seq + 1];
  for (int c = cend - 1; c >= cbeg; --c) {
    const int row0 = a.plan.chunk_row0[c];
    const int len = a.plan.chunk_len[c];
    const int nrep = a.plan.chunk_nrep[c];
    const size_t blk = (size_t)c * H + h;
    const float* Gg = a.ws.Gam + blk * BC * D;
    const float* Pg = a.ws.P + blk * BC * BC;
    const float* Tg = a.ws.T + blk * BC * BC;
    __syncthreads();
    const int save = a.plan.chunk_save[c];
    if (save >= 0) {
      const int p0 = a.plan.buf_cons_ptr[save], p1 = a.plan.buf_cons_ptr[save + 1];
      for (int e = tid; e < D * DVS; e += BT) {
        const int r = e / DVS, cc = e % DVS;
        float acc = s.DH[r][cc];
        for (int pi = p0; pi < p1; ++pi) {
          const int cs = a.plan.buf_cons[pi];
          acc += a.slot[((size_t)cs * H + h) * DD + (size_t)r * D + v0 + cc];
        }
        s.DH[r][cc] = acc;
        if (a.dh_boundary) a.dh_boundary[((size_t)save * H + h) * DD + (size_t)r * D + v0 + cc] = acc;
      }
    }
    {
      float* dst = a.dhc + blk * DD;
      for (int e = tid; e < D * DVS; e += BT) {
        const int r = e / DVS, cc = e % DVS;
        dst[(size_t)r * D + v0 + cc] = s.DH[r][cc];
      }
    }
    for (int e = tid; e < BC * DVS; e += BT) {
      const int i = e / DVS, cc = e % DVS;
      float x = 0.f;
      if (i >= nrep && i < len) {
        const int orow = a.plan.out_row[row0 + i];
        x = ld_in(dO, ((size_t)orow * H + h) * D + v0 + cc);
      }
      s.DO[i][cc] = x;
    }
    for (int e = tid; e < BC * BC; e += BT) s.P[e / BC][e % BC] = Pg[e];
    for (int e = tid; e < BC * D; e += BT) {
      const int i = e / D, ch = e % D;
      float kv = 0.f;
      if (i < len) {
        const int r = a.plan.row_index[row0 + i];
        kv = ld_in(k, ((size_t)r * H + h) * D + ch) * __expf(Gg[(BC - 1) * D + ch] - Gg[e]);
      }
      s.M[i][ch] = kv;
    }
    for (int ch = tid; ch < D; ch += BT) s.GC[ch] = __expf(Gg[(BC - 1) * D + ch]);
    __syncthreads();
    // ddelta = scale P^T dO + (K e^(Gam_C-Gam)) dh'
    gemm3<BC, DVS, BC + D, BW>(
        [&](int j, int kk) { return kk < BC ? sc * s.P[kk][j] : s.M[j][kk - BC]; },
        [&](int kk, int cc) { return kk < BC ? s.DO[kk][cc] : s.DH[kk - BC][cc]; },
        [&](int j, int cc, float x) { s.DD[j][cc] = x; });
    __syncthreads();
    for (int e = tid; e < BC * BC; e += BT) s.P[e / BC][e % BC] = Tg[e];
    __syncthreads();
    // dy = T^T ddelta
    gemm3<BC, DVS, BC, BW>(
        [&](int j, int i) { return s.P[i][j]; },
        [&](int i, int cc) { return s.DD[i][cc]; },
        [&](int j, int cc, float x) {
          s.DY[j][cc] = x;
          if (j < len) a.dy[((size_t)(row0 + j) * H + h) * D + v0 + cc] = x;
        },
        [](int j0, int, int kb) { return kb + 31 < j0; });
    // Q e^Gam
    for (int e = tid; e < BC * D; e += BT) {
      const int i = e / D, ch = e % D;
      float qv = 0.f;
      if (i < len) {
        const int r = a.plan.row_index[row0 + i];
        qv = ld_in(q, ((size_t)r * H + h) * D + ch) * __expf(Gg[e]);
      }
      s.M[i][ch] = qv;
    }
    __syncthreads();
    // dh = e^Gam_C dh' + scale (Q e^Gam)^T dO
    gemm3<D, DVS, BC, BW>(
        [&](int ch, int i) { return sc * s.M[i][ch]; },
        [&](int i, int cc) { return s.DO[i][cc]; },
        [&](int ch, int cc, float x) { s.DH[ch][cc] = s.GC[ch] * s.DH[ch][cc] + x; });
    __syncthreads();
    // diag(beta) K e^Gam
    for (int e = tid; e < BC * D; e += BT) {
      const int i = e / D, ch = e % D;
      float kv = 0.f;
      if (i < len) {
        const int r = a.plan.row_index[row0 + i];
        const size_t off = ((size_t)r * H + h) * D + ch;
        kv = a.beta[(size_t)r * H + h] * ld_in(k, off) * __expf(Gg[e]);
      }
      s.M[i][ch] = kv;
    }
    __syncthreads();
    // dh -= (diag(beta) K e^Gam)^T dy
    gemm3<D, DVS, BC, BW>(
        [&](int ch, int j) { return s.M[j][ch]; },
        [&](int j, int cc) { return s.DY[j][cc]; },
        [&](int ch, int cc, float x) { s.DH[ch][cc] -= x; });
  }
  __syncthreads();
  {
    float* dst = a.slot + ((size_t)seq * H + h) * DD;
    for (int e = tid; e < D * DVS; e += BT) {
      const int r = e / DVS, cc = e % DVS;
      dst[(size_t)r * D + v0 + cc] = s.DH[r][cc];
    }
  }
}

// ---------------------------------------------------------------------------
// chunk-local gradients
// ---------------------------------------------------------------------------

// destination of a row gradient: the output row, or the replay slot
__device__ inline float* grad_row(const BwdArgs& a, float* base, float* rep, int c, int i,
                                  int nrep, int row0, int h, int width) {
  if (i < nrep) return rep + ((size_t)(a.plan.chunk_rep0[c] + i) * a.H + h) * width;
  return base + ((size_t)a.plan.out_row[row0 + i] * a.H + h) * width;
}

template <int BC, int D>
struct DeltaSmem {
  float Hs[D][D + 1];
  float W[BC][D + 1];
};

// delta = U - W h, written over U
template <int BC, int D>
__global__ __launch_bounds__(BT) void k_gdelta(BwdArgs a) {
  __shared__ DeltaSmem<BC, D> s;
  const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const size_t blk = (size_t)c * a.H + h;
  const float* hs = a.chunk_h + blk * D * D;
  const float* Wg = a.ws.W + blk * BC * D;
  float* Ug = a.ws.U + blk * BC * D;
  for (int e = tid; e < D * D; e += BT) s.Hs[e / D][e % D] = hs[e];
  for (int e = tid; e < BC * D; e += BT) s.W[e / D][e % D] = Wg[e];
  __syncthreads();
  gemm3<BC, D, D, BW>(
      [&](int i, int ch) { return s.W[i][ch]; },
      [&](int ch, int cc) { return s.Hs[ch][cc]; },
      [&](int i, int cc, float x) { Ug[i * D + cc] -= x; });
}

template <int BC, int D>
struct HProdSmem {
  float Hs[D][D + 1];
  float X1[BC][D + 1];
  float X2[BC][D + 1];
  float beta[BC];
};

// dQt = scale dO h^T, dKt = -diag(beta) dy h^T, X = (K e^Gam) h
template <typename TIn, int BC, int D>
__global__ __launch_bounds__(BT) void k_ghprod(BwdArgs a) {
  __shared__ HProdSmem<BC, D> s;
  const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int H = a.H;
  const size_t blk = (size_t)c * H + h;
  const int row0 = a.plan.chunk_row0[c], len = a.plan.chunk_len[c], nrep = a.plan.chunk_nrep[c];
  const TIn* dO = (const TIn*)a.dO;
  const TIn* k = (const TIn*)a.k;
  const float* Gg = a.ws.Gam + blk * BC * D;
  const float* hs = a.chunk_h + blk * D * D;
  const float sc = a.scale;
  for (int e = tid; e < D * D; e += BT) s.Hs[e / D][e % D] = hs[e];
  for (int e = tid; e < BC * D; e += BT) {
    const int i = e / D, cc = e % D;
    float x = 0.f, y = 0.f;
    if (i < len) {
      if (i >= nrep) x = ld_in(dO, ((size_t)a.plan.out_row[row0 + i] * H + h) * D + cc);
      y = a.dy[((size_t)(row0 + i) * H + h) * D + cc];
    }
    s.X1[i][cc] = x;
    s.X2[i][cc] = y;
  }
  if (tid < BC) s.beta[tid] = tid < len ? a.beta[(size_t)a.plan.row_index[row0 + tid] * H + h] : 0.f;
  __syncthreads();
  float* dQt = a.gw.dQt + blk * BC * D;
  float* dKt = a.gw.dKt + blk * BC * D;
  float* X = a.gw.X + blk * BC * D;
  gemm3<BC, D, D, BW>(
      [&](int i, int cc) { return sc * s.X1[i][cc]; },
      [&](int cc, int ch) { return s.Hs[ch][cc]; },
      [&](int i, int ch, float x) { dQt[i * D + ch] = x; });
  gemm3<BC, D, D, BW>(
      [&](int i, int cc) { return -s.beta[i] * s.X2[i][cc]; },
      [&](int cc, int ch) { return s.Hs[ch][cc]; },
      [&](int i, int ch, float x) { dKt[i * D + ch] = x; });
  __syncthreads();
  for (int e = tid; e < BC * D; e += BT) {
    const int i = e / D, ch = e % D;
    float kv = 0.f;
    if (i < len) kv = ld_in(k, ((size_t)a.plan.row_index[row0 + i] * H + h) * D + ch) * __expf(Gg[e]);
    s.X1[i][ch] = kv;
  }
  __syncthreads();
  gemm3<BC, D, D, BW>(
      [&](int i, int ch) { return s.X1[i][ch]; },
      [&](int ch, int cc) { return s.Hs[ch][cc]; },
      [&](int i, int cc, float x) { X[i * D + cc] = x; });
}

template <int BC, int D>
struct DHProdSmem {
  float DHc[D][D + 1];
  float Del[BC][D + 1];
};

// dKh = delta dh'^T, deGC = rowsum(h * dh')
template <int BC, int D>
__global__ __launch_bounds__(BT) void k_gdhprod(BwdArgs a) {
  __shared__ DHProdSmem<BC, D> s;
  const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const size_t blk = (size_t)c * a.H + h;
  const float* dhc = a.dhc + blk * D * D;
  const float* hs = a.chunk_h + blk * D * D;
  const float* Del = a.ws.U + blk * BC * D;
  for (int e = tid; e < D * D; e += BT) s.DHc[e / D][e % D] = dhc[e];
  for (int e = tid; e < BC * D; e += BT) s.Del[e / D][e % D] = Del[e];
  __syncthreads();
  float* dKh = a.gw.dKh + blk * BC * D;
  gemm3<BC, D, D, BW>(
      [&](int j, int cc) { return s.Del[j][cc]; },
      [&](int cc, int ch) { return s.DHc[ch][cc]; },
      [&](int j, int ch, float x) { dKh[j * D + ch] = x; });
  for (int ch = tid; ch < D; ch += BT) {
    float acc = 0.f;
    for (int cc = 0; cc < D; ++cc) acc += hs[(size_t)ch * D + cc] * s.DHc[ch][cc];
    a.gw.deGC[blk * D + ch] = acc;
  }
}

template <int BC, int D>
struct SmallSmem {
  float DO[BC][D + 1];
  float DY[BC][D + 1];
  float Del[BC][D + 1];
  float A[BC][BC + 1];
  float beta[BC];
};

// dP, dA, dbeta, dv
template <typename TIn, int BC, int D>
__global__ __launch_bounds__(BT) void k_gsmall(BwdArgs a) {
  __shared__ SmallSmem<BC, D> s;
  const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int H = a.H;
  const size_t blk = (size_t)c * H + h;
  const int row0 = a.plan.chunk_row0[c], len = a.plan.chunk_len[c], nrep = a.plan.chunk_nrep[c];
  const TIn* dO = (const TIn*)a.dO;
  const TIn* v = (const TIn*)a.v;
  const float* Del = a.ws.U + blk * BC * D;
  const float* Ag = a.ws.A + blk * BC * BC;
  const float* X = a.gw.X + blk * BC * D;
  const float sc = a.scale;
  for (int e = tid; e < BC * D; e += BT) {
    const int i = e / D, cc = e % D;
    float x = 0.f, y = 0.f;
    if (i < len) {
      if (i >= nrep) x = ld_in(dO, ((size_t)a.plan.out_row[row0 + i] * H + h) * D + cc);
      y = a.dy[((size_t)(row0 + i) * H + h) * D + cc];
    }
    s.DO[i][cc] = x;
    s.DY[i][cc] = y;
    s.Del[i][cc] = Del[e];
  }
  for (int e = tid; e < BC * BC; e += BT) s.A[e / BC][e % BC] = Ag[e];
  if (tid < BC) s.beta[tid] = tid < len ? a.beta[(size_t)a.plan.row_index[row0 + tid] * H + h] : 0.f;
  __syncthreads();
  float* dP = a.gw.dP + blk * BC * BC;
  float* dA = a.gw.dA + blk * BC * BC;
  gemm3<BC, BC, D, BW>(
      [&](int i, int cc) { return sc * s.DO[i][cc]; },
      [&](int cc, int j) { return s.Del[j][cc]; },
      [&](int i, int j, float x) { dP[i * BC + j] = (j <= i) ? x : 0.f; });
  gemm3<BC, BC, D, BW>(
      [&](int i, int cc) { return -s.beta[i] * s.DY[i][cc]; },
      [&](int cc, int j) { return s.Del[j][cc]; },
      [&](int i, int j, float x) { dA[i * BC + j] = (j < i) ? x : 0.f; });
  __syncthreads();
  // per element: dy * (v - X - A delta), into DO
  gemm3<BC, D, BC, BW>(
      [&](int i, int j) { return s.A[i][j]; },
      [&](int j, int cc) { return s.Del[j][cc]; },
      [&](int i, int cc, float x) {
        float vv = 0.f;
        if (i < len) vv = ld_in(v, ((size_t)a.plan.row_index[row0 + i] * H + h) * D + cc);
        s.DO[i][cc] = s.DY[i][cc] * (vv - X[i * D + cc] - x);
      },
      [](int i0, int, int kb) { return kb > i0 + 15; });
  __syncthreads();
  if (tid < len) {
    float acc = 0.f;
    for (int cc = 0; cc < D; ++cc) acc += s.DO[tid][cc];
    *grad_row(a, a.dbeta, a.rep_db, c, tid, nrep, row0, h, 1) = acc;
  }
  for (int e = tid; e < BC * D; e += BT) {
    const int i = e / D, cc = e % D;
    if (i < len) grad_row(a, a.dv, a.rep_dv, c, i, nrep, row0, h, D)[cc] = s.beta[i] * s.DY[i][cc];
  }
}

template <int BC, int D>
struct FinalSmem {
  float K[BC][D + 1];
  float Q[BC][D + 1];
  float G[BC][D + 1];
  union {
    struct {
      float dP[BC][BC + 1];
      float dA[BC][BC + 1];
    } pa;
    float dG[BC][D + 1];
  } u;
  float colsum[D];
};

// Decay-weighted products of dP and dA with q and k, then dq, dk, dg.
//   dqP_ic  = sum_{j<=i} dP_ij k_jc e^(Gam_ic-Gam_jc)    dkP_jc  = sum_{i>=j} dP_ij q_ic e^(..)
//   dkAr_ic = sum_{j< i} dA_ij k_jc e^(..)               dkAc_jc = sum_{i> j} dA_ij k_ic e^(..)
// Wave w owns the rows of 16-row block w: it forms the row-side sums of its
// block (pairs (w, J), J <= w) and the column-side sums (pairs (I, w), I >= w),
// each pair through the reference m = Gam at the first row of the column
// block (as in the forward), so that every factor stays bounded.
template <typename TIn, int BC, int D>
__global__ __launch_bounds__(BT) void k_gfinal(BwdArgs a) {
  __shared__ FinalSmem<BC, D> s;
  constexpr int NB = BC / 16;
  constexpr int NCT = D / 16;
  const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int H = a.H;
  const size_t blk = (size_t)c * H + h;
  const int row0 = a.plan.chunk_row0[c], len = a.plan.chunk_len[c], nrep = a.plan.chunk_nrep[c];
  const TIn* q = (const TIn*)a.q;
  const TIn* k = (const TIn*)a.k;
  const float* Gg = a.ws.Gam + blk * BC * D;
  const float* dPg = a.gw.dP + blk * BC * BC;
  const float* dAg = a.gw.dA + blk * BC * BC;
  const float* dQt = a.gw.dQt + blk * BC * D;
  const float* dKt = a.gw.dKt + blk * BC * D;
  const float* dKh = a.gw.dKh + blk * BC * D;
  const float* deGC = a.gw.deGC + blk * D;
  for (int e = tid; e < BC * D; e += BT) {
    const int i = e / D, ch = e % D;
    float kv = 0.f, qv = 0.f;
    if (i < len) {
      const size_t off = ((size_t)a.plan.row_index[row0 + i] * H + h) * D + ch;
      kv = ld_in(k, off);
      qv = ld_in(q, off);
    }
    s.K[i][ch] = kv;
    s.Q[i][ch] = qv;
    s.G[i][ch] = Gg[e];
  }
  for (int e = tid; e < BC * BC; e += BT) {
    s.u.pa.dP[e / BC][e % BC] = dPg[e];
    s.u.pa.dA[e / BC][e % BC] = dAg[e];
  }
  __syncthreads();
  // column sums for the Gam_C terms: sum_j dKh_jc * K_jc e^(Gam_C - Gam_jc)
  for (int ch = tid; ch < D; ch += BT) {
    float acc = 0.f;
    const float gc = s.G[BC - 1][ch];
    for (int j = 0; j < BC; ++j) acc += dKh[j * D + ch] * s.K[j][ch] * __expf(gc - s.G[j][ch]);
    s.colsum[ch] = acc + deGC[ch] * __expf(gc);
  }

  const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, quad = lane >> 4;
  float rq[NCT][4], rk[NCT][4], rg[NCT][4];
#pragma unroll
  for (int t = 0; t < NCT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) rq[t][r] = rk[t][r] = rg[t][r] = 0.f;

  if (wave < NB) {
    const int B0 = 16 * wave;  // first row of this wave's block
    // --- row side: pairs (wave, J), J <= wave ---
    for (int J = 0; J <= wave; ++J) {
      const int mrow = 16 * J;
#pragma unroll
      for (int t = 0; t < NCT; ++t) {
        const int c0 = 16 * t;
        // A operands: dP[B0+i][16J+j], dA[..] (k = j in 0..15; lanes quad>=2 carry zeros)
        bf16x8 ph, pl, ah, al, bh, bl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int jj = quad * 8 + e;
          float pv = 0.f, av = 0.f, bv = 0.f;
          if (jj < 16) {
            pv = s.u.pa.dP[B0 + l16][16 * J + jj];
            av = s.u.pa.dA[B0 + l16][16 * J + jj];
            const int ch = c0 + l16;
            bv = s.K[16 * J + jj][ch] * __expf(s.G[mrow][ch] - s.G[16 * J + jj][ch]);
          }
          __bf16 hh, ll;
          split_bf16(pv, hh, ll); ph[e] = hh; pl[e] = ll;
          split_bf16(av, hh, ll); ah[e] = hh; al[e] = ll;
          split_bf16(bv, hh, ll); bh[e] = hh; bl[e] = ll;
        }
        f32x4 accP = {0.f, 0.f, 0.f, 0.f}, accA = {0.f, 0.f, 0.f, 0.f};
        accP = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, bh, accP, 0, 0, 0);
        accP = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, bl, accP, 0, 0, 0);
        accP = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, bh, accP, 0, 0, 0);
        accA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, accA, 0, 0, 0);
        accA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, accA, 0, 0, 0);
        accA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, accA, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = B0 + quad * 4 + r, ch = c0 + l16;
          const float f = __expf(s.G[i][ch] - s.G[mrow][ch]);
          const float vp = accP[r] * f, va = accA[r] * f;
          rq[t][r] += vp;
          rk[t][r] += va;
          rg[t][r] += s.Q[i][ch] * vp + s.K[i][ch] * va;
        }
      }
    }
    // --- column side: pairs (I, wave), I >= wave ---
    for (int I = wave; I < NB; ++I) {
      const int mrow = B0;
#pragma unroll
      for (int t = 0; t < NCT; ++t) {
        const int c0 = 16 * t;
        // A operands: dP^T[B0+j][16I+i]; B operands: q / k rows of block I, decayed
        bf16x8 ph, pl, ah, al, qh, ql, kh, kl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int ii = quad * 8 + e;
          float pv = 0.f, av = 0.f, qv = 0.f, kv = 0.f;
          if (ii < 16) {
            pv = s.u.pa.dP[16 * I + ii][B0 + l16];
            av = s.u.pa.dA[16 * I + ii][B0 + l16];
            const int ch = c0 + l16;
            const float f = __expf(s.G[16 * I + ii][ch] - s.G[mrow][ch]);
            qv = s.Q[16 * I + ii][ch] * f;
            kv = s.K[16 * I + ii][ch] * f;
          }
          __bf16 hh, ll;
          split_bf16(pv, hh, ll); ph[e] = hh; pl[e] = ll;
          split_bf16(av, hh, ll); ah[e] = hh; al[e] = ll;
          split_bf16(qv, hh, ll); qh[e] = hh; ql[e] = ll;
          split_bf16(kv, hh, ll); kh[e] = hh; kl[e] = ll;
        }
        f32x4 accP = {0.f, 0.f, 0.f, 0.f}, accA = {0.f, 0.f, 0.f, 0.f};
        accP = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, qh, accP, 0, 0, 0);
        accP = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, ql, accP, 0, 0, 0);
        accP = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, qh, accP, 0, 0, 0);
        accA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, kh, accA, 0, 0, 0);
        accA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, kl, accA, 0, 0, 0);
        accA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, kh, accA, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = B0 + quad * 4 + r, ch = c0 + l16;
          const float f = __expf(s.G[mrow][ch] - s.G[j][ch]);
          const float vp = accP[r] * f, va = accA[r] * f;
          rk[t][r] += vp + va;
          rg[t][r] -= s.K[j][ch] * (vp + va);
        }
      }
    }
  }
  __syncthreads();  // dP / dA no longer read; dG reuses their space
  if (wave < NB) {
    const int B0 = 16 * wave;
#pragma unroll
    for (int t = 0; t < NCT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = B0 + quad * 4 + r, ch = 16 * t + l16;
        const float Gi = s.G[i][ch];
        const float eg = __expf(Gi);
        const float ek = __expf(s.G[BC - 1][ch] - Gi);
        const float dqt = dQt[i * D + ch], dkt = dKt[i * D + ch], dkh = dKh[i * D + ch];
        const float qi = s.Q[i][ch], ki = s.K[i][ch];
        const float dq = dqt * eg + rq[t][r];
        const float dk = dkt * eg + dkh * ek + rk[t][r];
        float dG = dqt * qi * eg + dkt * ki * eg - dkh * ki * ek + rg[t][r];
        if (i == BC - 1) dG += s.colsum[ch];
        s.u.dG[i][ch] = dG;
        if (i < len) {
          grad_row(a, a.dq, a.rep_dq, c, i, nrep, row0, h, D)[ch] = dq;
          grad_row(a, a.dk, a.rep_dk, c, i, nrep, row0, h, D)[ch] = dk;
        }
      }
  }
  __syncthreads();
  // dg = reverse cumulative sum of dGam over the chunk's rows
  for (int ch = tid; ch < D; ch += BT) {
    float acc = 0.f;
    for (int i = BC - 1; i >= 0; --i) {
      acc += s.u.dG[i][ch];
      if (i < len) grad_row(a, a.dg, a.rep_dg, c, i, nrep, row0, h, D)[ch] = acc;
    }
  }
}

// replayed-row gradients added into their compact rows (fixed order)
template <int D>
__global__ __launch_bounds__(BT) void k_reduce_rep(BwdArgs a) {
  const int e = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int H = a.H;
  const int row = a.plan.rep_row[e];
  const int p0 = a.plan.rep_ptr[e], p1 = a.plan.rep_ptr[e + 1];
  for (int ch = tid; ch < D; ch += BT) {
    const size_t o = ((size_t)row * H + h) * D + ch;
    float sq = a.dq[o], sk = a.dk[o], sg = a.dg[o], sv = a.dv[o];
    for (int p = p0; p < p1; ++p) {
      const size_t r = ((size_t)a.plan.rep_slot[p] * H + h) * D + ch;
      sq += a.rep_dq[r];
      sk += a.rep_dk[r];
      sg += a.rep_dg[r];
      sv += a.rep_dv[r];
    }
    a.dq[o] = sq;
    a.dk[o] = sk;
    a.dg[o] = sg;
    a.dv[o] = sv;
  }
  if (tid == 0) {
    float sb = a.dbeta[(size_t)row * H + h];
    for (int p = p0; p < p1; ++p) sb += a.rep_db[(size_t)a.plan.rep_slot[p] * H + h];
    a.dbeta[(size_t)row * H + h] = sb;
  }
}

// dh0 of every root: sum of the start gradients of its sequences (fixed order)
template <int D>
__global__ __launch_bounds__(BT) void k_reduce_dh0(BwdArgs a) {
  const int rt = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int H = a.H;
  const int p0 = a.plan.root_seq_ptr[rt], p1 = a.plan.root_seq_ptr[rt + 1];
  const size_t DD = (size_t)D * D;
  for (int e = tid; e < D * D; e += BT) {
    float acc = 0.f;
    for (int p = p0; p < p1; ++p) acc += a.slot[((size_t)a.plan.root_seq[p] * H + h) * DD + e];
    a.dh0[((size_t)rt * H + h) * DD + e] = acc;
  }
}

template <typename TIn, int BC, int D>
hipError_t launch_bwd_t(const BwdArgs& a, const FwdArgs& pa, int n_chunks,
                        const int* round_ptr_host, int n_rounds, int n_rep_rows, int n_root,
                        hipStream_t st) {
  hipError_t e;
#define KDA_CHECK()                      \
  e = hipGetLastError();                 \
  if (e != hipSuccess) return e;
  const dim3 cg(n_chunks, a.H);
  if (n_chunks > 0) {
    KDA_LAUNCH("kda_chunk_prep", (k_prep<TIn, BC, D>), cg, dim3(BT), st, pa);
    KDA_CHECK();
  }
  e = launch_bwd_rounds(a, sizeof(TIn) == 2, BC, D, round_ptr_host, n_rounds, st);
  if (e != hipSuccess) return e;
  if (n_chunks > 0) {
    KDA_LAUNCH("kda_bwd_delta", (k_gdelta<BC, D>), cg, dim3(BT), st, a);
    KDA_CHECK();
    KDA_LAUNCH("kda_bwd_hprod", (k_ghprod<TIn, BC, D>), cg, dim3(BT), st, a);
    KDA_CHECK();
    KDA_LAUNCH("kda_bwd_dhprod", (k_gdhprod<BC, D>), cg, dim3(BT), st, a);
    KDA_CHECK();
    KDA_LAUNCH("kda_bwd_small", (k_gsmall<TIn, BC, D>), cg, dim3(BT), st, a);
    KDA_CHECK();
    KDA_LAUNCH("kda_bwd_final", (k_gfinal<TIn, BC, D>), cg, dim3(BT), st, a);
    KDA_CHECK();
  }
  if (n_rep_rows > 0) {
    KDA_LAUNCH("kda_bwd_reduce_replay", (k_reduce_rep<D>), dim3(n_rep_rows, a.H), dim3(BT), st, a);
    KDA_CHECK();
  }
  if (n_root > 0) {
    KDA_LAUNCH("kda_bwd_reduce_dh0", (k_reduce_dh0<D>), dim3(n_root, a.H), dim3(BT), st, a);
    KDA_CHECK();
  }
#undef KDA_CHECK
  return hipSuccess;
}

hipError_t launch_bwd(const BwdArgs& a, const FwdArgs& pa, bool bf16, int BC, int D,
                      int n_chunks, const int* round_ptr_host, int n_rounds, int n_rep_rows,
                      int n_root, hipStream_t st) {
#define KDA_BWD_CASE(T, BCv, Dv)                                                            \
  if (BC == BCv && D == Dv)                                                                 \
    return launch_bwd_t<T, BCv, Dv>(a, pa, n_chunks, round_ptr_host, n_rounds, n_rep_rows, \
                                    n_root, st);
  if (bf16) {
    KDA_BWD_CASE(uint16_t, 64, 128)
    KDA_BWD_CASE(uint16_t, 64, 64)
    KDA_BWD_CASE(uint16_t, 16, 128)
    KDA_BWD_CASE(uint16_t, 16, 64)
  } else {
    KDA_BWD_CASE(float, 64, 128)
    KDA_BWD_CASE(float, 64, 64)
    KDA_BWD_CASE(float, 16, 128)
    KDA_BWD_CASE(float, 16, 64)
  }
#undef KDA_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace kda
