// kda_grad.hip -- chunk-local gradients of every chunk (gfx950).
//
// One block (8 waves) per (chunk, head), after the state-gradient rounds.  With
// h the chunk's start state (saved by the forward), dh' its end-state gradient
// and dy (kda_bwd.hip), and A, Td and V from the chunk's forward image:
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
// Layout of the work.  Every global load of the block is issued first.  Phase 1:
// wave w owns a 16-column block of dv (Z, delta, dbeta and deGC partials,
// dv), with dO, -dZ, delta and h staged in LDS as fp16.  Phase 2: wave w owns
// the 16-row block tI = w % NB of the chunk and, transposed ([channel][row]),
// the output tiles (C, tI) with C = w / NB + (8 / NB) m; it forms dQt^T, dKt^T,
// dKh^T for them, and the dP / dA blocks that its row block meets -- (tI, J),
// J <= tI as [j][i] tiles and (I, tI), I >= tI as [i][j] tiles -- which stay in
// registers as hi/lo bf16 B operands (an accumulator tile is a B fragment of
// the 16x16x16 matrix-core op).  Phase 3, per 64-channel pass: the decay
// factored q / k operands are staged transposed, the decay-weighted products
// run on hi/lo bf16 matrix cores (each block pair around the first row of its
// column block, the channel factor between the two references applied to the
// output rows), the gradients are combined, and dg is formed by a parallel
// reverse scan.
//
// Chunks with decays past the range of the factored products (a row more than
// kExactDecay below its block's first row, or a single step of more than
// kExactStep) run phase 3 on exact per-pair exponentials instead
// (phase3_exact_*): any gate g <= 0 is supported.
#include <type_traits>

#include "chunk.h"
#include "timing.h"

namespace kda {

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ inline f32x4 mfmab16(const s16x4& a, const s16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ inline short bf16_bits(__bf16 x) { return __builtin_bit_cast(short, x); }
__device__ inline float bf16_val(__bf16 x) { return (float)x; }
// accumulator tile -> hi/lo bf16 B fragment of the 16x16x16 op
__device__ inline void split_tile(const f32x4& t, s16x4& hi, s16x4& lo) {
  bf16x2 h0, l0, h1, l1;
  split_bf16x2(t[0], t[1], h0, l0);
  split_bf16x2(t[2], t[3], h1, l1);
  hi = __builtin_bit_cast(s16x4, __builtin_shufflevector(h0, h1, 0, 1, 2, 3));
  lo = __builtin_bit_cast(s16x4, __builtin_shufflevector(l0, l1, 0, 1, 2, 3));
}
// the hi/lo product  ah bh + ah bl + al bh
__device__ inline f32x4 mma3(const s16x4& ah, const s16x4& al, const s16x4& bh, const s16x4& bl) {
  f32x4 t = {0.f, 0.f, 0.f, 0.f};
  t = mfmab16(ah, bh, t);
  t = mfmab16(ah, bl, t);
  t = mfmab16(al, bh, t);
  return t;
}

template <int BC, int D>
struct GradGeom {
  static constexpr int NB = BC / 16;             // 16-row blocks of the chunk
  static constexpr int NCB = D / 16;             // 16-channel blocks
  static constexpr int KD = D / 32;              // 32-deep k steps over a head dim
  static constexpr int NHF = D / 64;             // 64-channel passes of phase 3
  static constexpr int NS = NB + 1;              // dP / dA blocks met by one row block
  static constexpr int NG = NW / NB;             // waves per row block
  static constexpr int NTW = (NCB / NG) > 0 ? NCB / NG : 1;  // output tiles per wave
  static constexpr int PD = D + 8;               // fp16 [*][D] pitch
  static constexpr int PB = BC + 12;             // 16-bit [*][BC] pitch: 8-byte fragment reads by 16
                                                 // rows hit distinct banks (rows 8-byte aligned)
  static constexpr int PG = BC + 1;              // fp32 [64][BC] pitch
  static constexpr int NLOW = NB * (NB + 1) / 2; // lower block pairs
  static constexpr int DH = 64;
  static constexpr int NRG = NT / DH;            // row groups of the element mapping
  static constexpr int RPT = BC / NRG;           // rows per thread in the element mapping
  static_assert(RPT >= 1 && NCB % 4 == 0, "geometry");
};

// eight bf16 values as two 8-byte stores (rows of the [*][PB] arrays are
// 8-byte aligned)
__device__ inline void put8(__bf16* p, const bf16x8& v) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  *(bf16x4*)p = (bf16x4){v[0], v[1], v[2], v[3]};
  *(bf16x4*)(p + 4) = (bf16x4){v[4], v[5], v[6], v[7]};
}

// lower block pair (I, J), J <= I -> I (I + 1) / 2 + J
__device__ inline int low_index(int I, int J) { return I * (I + 1) / 2 + J; }

template <int BC, int D>
struct GradSmem {
  using G = GradGeom<BC, D>;
  union {
    struct {                       // phases 1-2
      _Float16 A[BC][G::PB];       // -A (strict lower), as the image holds it
      _Float16 Td[BC][24];         // diagonal-block inverses
      union {
        _Float16 Kn[BC][G::PD];    // -(K e^Gam)        [i][c], until Z is formed
        _Float16 dO[BC][G::PD];    // scale dO          [i][v]
      } x;
      _Float16 nZ[BC][G::PD];      // -diag(beta) dy    [i][v]
      _Float16 dl[BC][G::PD];      // delta             [j][v]
      _Float16 Hs[D][G::PD];       // h, later dh'      [c][v]
    } p;
    struct {                       // phase 3, one 64-channel pass, transposed
      __bf16 rh[64][G::PB], rl[64][G::PB];   // K e^(gref - Gam)   [c][j]
      __bf16 qh[64][G::PB], ql[64][G::PB];   // Q e^(Gam - gref)   [c][i]
      __bf16 kh[64][G::PB], kl[64][G::PB];   // K e^(Gam - gref)   [c][i]
      float gam[64][G::PG];                  // Gam, replaced by dGam
      __bf16 qraw[64][G::PB], kraw[64][G::PB];  // Q, K as read (bf16 inputs)  [c][i]
    } d;
    struct {                       // phase 3 of a chunk with exact pairs (decays past the
                                   // factored range), one 64-channel pass, transposed
      float dgam[64][G::PG];       // dGam of the pass           [c][i]
      float gam[64][G::PG];        // Gam                        [c][i]
      float qf[64][G::PG], kf[64][G::PG];   // q, k as read     [c][i]
      float dP[BC][G::PG], dA[BC][G::PG];   // dP, dA (lower)    [i][j]
    } e;
  } u;
  __attribute__((aligned(16))) float dfac[G::NLOW][D];   // e^(gref_I - gref_J), J <= I
  __attribute__((aligned(16))) float gref[G::NB][D];     // Gam at the first row of each block
  __attribute__((aligned(16))) float eref[G::NB][D];     // e^gref
  __attribute__((aligned(16))) float ecg[G::NB][D];      // e^(Gam_C - gref)
  float csum[G::NB][D];     // sum over a row block of dKh_jc K_jc e^(Gam_C - Gam_jc)
  float redb[NW][BC];       // dbeta partials per wave
  float redg[NW][D];        // deGC partials per wave
  float part[G::NRG][D];    // row-group sums (Gam, then the reverse scan)
  float degc[D];
  float gcl[D];             // Gam_C
  float beta[BC];
  int orow[BC];
  int irow[BC];   // input row of each chunk row (-1 past the chunk)
  int bad;        // some row's decay from its block's first row exceeds kExactDecay
};

// destination of a row gradient: the output row, or the replay slot
__device__ inline float* grad_dst(const BwdArgs& a, float* base, float* rep, int rep0, int orow,
                                  int i, int nrep, int h, int width) {
  if (i < nrep) return rep + ((size_t)(rep0 + i) * a.H + h) * width;
  return base + ((size_t)orow * a.H + h) * width;
}

// Phase 3 of a chunk with exact pairs: staging.  Channel c0 of pass hf, rows
// r0 .. r0 + RPT - 1: Gam, q and k as read; on the first pass the waves of
// the first column group also store their dP / dA blocks (tI, J <= tI) as
// fp32 [i][j] (hi + lo of the B fragments, the values the factored path
// uses; entries above the diagonal are never read).
template <int BC, int D, int NS, int NE>
__device__ inline void phase3_exact_stage(GradSmem<BC, D>& s, int hf, const float (&gm)[NE],
                                          const float (&qq)[NE], const float (&kk)[NE],
                                          const s16x4 (&Ph)[NS], const s16x4 (&Pl)[NS],
                                          const s16x4 (&Ah)[NS], const s16x4 (&Al)[NS], int tI,
                                          int tu) {
  using G = GradGeom<BC, D>;
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int c0 = tid % G::DH, r0 = (tid / G::DH) * G::RPT;
#pragma unroll
  for (int t = 0; t < G::RPT; ++t) {
    const int n = hf * G::RPT + t, i = r0 + t;
    s.u.e.gam[c0][i] = gm[n];
    s.u.e.qf[c0][i] = qq[n];
    s.u.e.kf[c0][i] = kk[n];
  }
  if (hf == 0 && tu == 0) {
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
      if (sl <= tI) {   // tile (tI, J = sl) as [j][i]: lane holds j = 16 sl + 4 g + r, i = 16 tI + l16
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        const int i = 16 * tI + l16;
        // whole-vector bit casts (a cast of one vector element is not used)
        const bf16x4 ph = __builtin_bit_cast(bf16x4, Ph[sl]), pl = __builtin_bit_cast(bf16x4, Pl[sl]);
        const bf16x4 ah = __builtin_bit_cast(bf16x4, Ah[sl]), al = __builtin_bit_cast(bf16x4, Al[sl]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * sl + 4 * g + r;
          s.u.e.dP[i][j] = bf16_val(ph[r]) + bf16_val(pl[r]);
          s.u.e.dA[i][j] = bf16_val(ah[r]) + bf16_val(al[r]);
        }
      }
    }
  }
}

// Phase 3 of a chunk with exact pairs: the decay-weighted sums and the
// combine of output tile C (channels 16 C ..) x row block tI, lane element
// (channel 16 C + 4 g + r, row i = 16 tI + l16):
//   rowP = sum_{j<i} dP_ij k_j e^(Gam_i-Gam_j)    rowA = sum_{j<i} dA_ij k_j e^(..)
//   colP = sum_{j>i} dP_ji q_j e^(Gam_j-Gam_i)    colA = sum_{j>i} dA_ji k_j e^(..)
// every exponent negative, and the pair (i, i) (factor 1) apart; then dq, dk
// and dGam as in the factored path.  Terms whose decay spans no row -- the
// pair (i, i) on both sides, and k e^(Gam_C - Gam) of the chunk's last row
// against the Gam_C term -- cancel exactly in dGam and are left out of it:
// with decays this strong dg itself is tiny, and their rounding would swamp it.
template <int BC, int D>
__device__ inline void phase3_exact_tile(const BwdArgs& a, GradSmem<BC, D>& s, int hf, int C,
                                         int tI, const f32x4& dQt, const f32x4& dKt,
                                         const f32x4& dKh, int rep0, int nrep, int len, int h,
                                         float inv) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
  const int cb = 16 * (C % 4), cf = 64 * hf + cb + 4 * g;
  const int i = 16 * tI + l16;
  float4 vq, vk;
  float cs[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int cl = cb + 4 * g + r;
    const float* Gc = &s.u.e.gam[cl][0];
    const float* Kc = &s.u.e.kf[cl][0];
    const float* Qc = &s.u.e.qf[cl][0];
    const float gi = Gc[i];
    float rowP = 0.f, rowA = 0.f, colP = 0.f, colA = 0.f;
    for (int j = 0; j < BC; ++j) {
      const float gj = Gc[j], kj = Kc[j], qj = Qc[j];
      const float E = __expf(j < i ? gi - gj : gj - gi);
      const float pr = s.u.e.dP[i][j], ar = s.u.e.dA[i][j];   // row side (j < i)
      const float pc = s.u.e.dP[j][i], ac = s.u.e.dA[j][i];   // column side (j > i)
      rowP += j < i ? pr * kj * E : 0.f;
      rowA += j < i ? ar * kj * E : 0.f;
      colP += j > i ? pc * qj * E : 0.f;
      colA += j > i ? ac * kj * E : 0.f;
    }
    const float ki = Kc[i], qi = Qc[i];
    const float dPii = s.u.e.dP[i][i];
    const float eg = __expf(gi), ec = __expf(s.gcl[cf + r] - gi);
    const float xq = dQt[r] * eg + rowP;
    const float xk = dKt[r] * eg + rowA;
    const float kh2 = i < len - 1 ? dKh[r] * ki * ec : 0.f;   // the last row's cancels
    cs[r] = kh2;
    s.u.e.dgam[cl][i] = qi * xq + ki * xk - kh2 - ki * (colP + colA);
    (&vq.x)[r] = xq + dPii * ki;
    (&vk.x)[r] = xk + dKh[r] * ec + colP + colA + dPii * qi;
  }
  if (i < len) {
    const int orow = s.orow[i];
    *(float4*)(grad_dst(a, a.dq, a.rep_dq, rep0, orow, i, nrep, h, D) + cf) =
        make_float4(inv * vq.x, inv * vq.y, inv * vq.z, inv * vq.w);
    *(float4*)(grad_dst(a, a.dk, a.rep_dk, rep0, orow, i, nrep, h, D) + cf) =
        make_float4(inv * vk.x, inv * vk.y, inv * vk.z, inv * vk.w);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float x = row_sum16(cs[r]);
    if (l16 == 0) s.csum[tI][cf + r] = x;
  }
}

// A chunk also takes the exact phase 3 when some row decays by more than this
// in one step: dg of such a row is of the order of e^-kExactStep times the
// terms whose rounding the factored sums would leave in it.
constexpr float kExactStep = 20.f;

template <typename TIn, int BC, int D>
__global__ __launch_bounds__(NT) void k_bwd_grad(BwdArgs a, int c_begin) {
  using G = GradGeom<BC, D>;
  constexpr int NB = G::NB, NCB = G::NCB, KD = G::KD, NHF = G::NHF, NS = G::NS;
  constexpr int NG = G::NG, NTW = G::NTW, DH = G::DH, NRG = G::NRG, RPT = G::RPT;
  constexpr int NE = RPT * NHF;
  constexpr int KB = (BC + 31) / 32;
  constexpr bool HALF = (BC == 16);
  constexpr int NV4 = (BC * D / 4 + NT - 1) / NT;   // 4-element pieces of dO per thread
  // bf16 inputs: the combine of phase 3 rebuilds the decayed q, k from the
  // inputs themselves (exact in bf16) instead of their hi/lo split products
  constexpr bool RAWQK = std::is_same<TIn, uint16_t>::value;
  __shared__ GradSmem<BC, D> s;
  const int c = c_begin + blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int H = a.H;
  const size_t blk = (size_t)c * H + h;
  const size_t DD = (size_t)D * D;
  const int row0 = ld_uni(a.plan.chunk_row0, c), len = ld_uni(a.plan.chunk_len, c);
  const int nrep = ld_uni(a.plan.chunk_nrep, c), rep0 = ld_uni(a.plan.chunk_rep0, c);
  const TIn* q = (const TIn*)a.q;
  const TIn* k = (const TIn*)a.k;
  const TIn* dOp = (const TIn*)a.dOp;
  const FwdImage<BC, D, TIn>* F =
      (const FwdImage<BC, D, TIn>*)(a.fimg + blk * fwd_image_bytes(BC, D));
  const int cround = ld_uni(a.plan.chunk_round, c);

  // ---- global loads, issued in the order of their first use: loads return
  // in issue order, so each phase waits only for what it reads while the
  // later ones are still in flight.  LDS writes and register layouts come
  // where they are needed. ----
  const int c0 = tid % DH, rg = tid / DH, r0 = rg * RPT;  // element mapping: channel c0 + 64 hf, rows r0 ..
  // the row indices are wave-uniform (a wave's lanes share rows r0 ..): scalar
  // loads, so that the input loads they address wait for no vector load
  const int r0w = __builtin_amdgcn_readfirstlane(r0);
  int rows[RPT];
#pragma unroll
  for (int t = 0; t < RPT; ++t) rows[t] = r0w + t < len ? ld_uni(a.plan.row_index, row0 + r0w + t) : -1;
  int trow = -1, torow = -1;  // row table entries (tid < BC)
  if (tid < BC && tid < len) {
    trow = a.plan.row_index[row0 + tid];
    torow = tid >= nrep ? a.plan.out_row[row0 + tid] : -1;
  }
  // g, then k, through this thread's row indices (Gam, K e^Gam)
  float gm[NE], kk[NE], qq[NE];
#pragma unroll
  for (int hf = 0; hf < NHF; ++hf)
#pragma unroll
    for (int t = 0; t < RPT; ++t) {
      const int r = rows[t];
      const float x = a.g[((size_t)(r < 0 ? 0 : r) * H + h) * D + c0 + DH * hf];
      gm[hf * RPT + t] = r >= 0 ? x : 0.f;
    }
#pragma unroll
  for (int hf = 0; hf < NHF; ++hf)
#pragma unroll
    for (int t = 0; t < RPT; ++t) {
      const int r = rows[t];
      const float y = ld_in(k, ((size_t)(r < 0 ? 0 : r) * H + h) * D + c0 + DH * hf);
      kk[hf * RPT + t] = r >= 0 ? y : 0.f;
    }
  // start state and V as accumulator pieces of their 16x16 tiles (phase 1),
  // A and Td of the forward image, beta
  const bool vw = wave < NCB;
  const int wv = vw ? wave : 0;   // column block the loads use (waves past D/16 load and drop one)
  const int col = 16 * wave + l16;
  f16x4 hraw[NCB], dhraw[NCB];
  f16x4 dyh[NB];
  f32x4 dyv[NB], z[NB];
  in4_t<TIn> vraw[NB];
  const _Float16* hsrc = a.chunk_h + blk * DD;
  const _Float16* dhsrc = a.dhc + blk * DD;
#pragma unroll
  for (int C = 0; C < NCB; ++C) hraw[C] = *(const f16x4*)(hsrc + state_tile<D>(C, wv));
#pragma unroll
  for (int J = 0; J < NB; ++J) vraw[J] = *(const in4_t<TIn>*)(&F->V[0][0] + state_tile<D>(J, wv));
  constexpr int NAV = (BC * BC / 4 + NT - 1) / NT;   // 8-byte pieces of A (swizzled rows)
  f16x4 av[NAV];
  f16x8 tv;
#pragma unroll
  for (int n = 0; n < NAV; ++n) {
    const int e = tid + NT * n, i = e / (BC / 4), j0 = (e % (BC / 4)) * 4;
    if (e < BC * BC / 4) av[n] = *(const f16x4*)&F->L[i][swz<BC>(i, j0)];
  }
  if (tid < BC * 2) tv = *(const f16x8*)&F->Td[tid / 2][(tid % 2) * 8];
  const float tbeta = trow >= 0 ? a.beta[(size_t)trow * H + h] : 0.f;
  // dy (phase 1), dO (after Z), the end-state gradient (end of phase 2); q
  // (phase 3) follows at the start of phase 1, which keeps the loads in
  // flight here within what one wait count can track (63)
#pragma unroll
  for (int J = 0; J < NB; ++J)   // (rows past the chunk are zeroed where used)
    dyh[J] = *(const f16x4*)&a.dy[blk * (BC * D) + state_tile<D>(J, wv)];
  // dO from the chunk's tiles (zero on replay rows and past the chunk):
  // piece e = tid + NT n is lane e % 64 of tile e / 64, one contiguous
  // 512- or 1024-byte run per wave
  // (no branch around a load: a branch that uses the loaded value makes the
  // compiler wait for every earlier load there)
  in4_t<TIn> dov[NV4];
#pragma unroll
  for (int n = 0; n < NV4; ++n) {
    const int e = tid + NT * n;
    const int ec = (BC * D / 4) % NT == 0 || e < BC * D / 4 ? e : BC * D / 4 - 1;
    dov[n] = *(const in4_t<TIn>*)&dOp[blk * (BC * D) + 4 * (size_t)ec];
  }
#pragma unroll
  for (int C = 0; C < NCB; ++C) dhraw[C] = *(const f16x4*)(dhsrc + state_tile<D>(C, wv));

  // ---- Gam: running sums per row group, then their prefix ----
  bool steep = false;   // a single row decays by more than kExactStep
#pragma unroll
  for (int hf = 0; hf < NHF; ++hf) {
    float run = 0.f;
#pragma unroll
    for (int t = 0; t < RPT; ++t) {
      steep |= gm[hf * RPT + t] < -kExactStep;
      run += gm[hf * RPT + t];
      gm[hf * RPT + t] = run;
    }
    s.part[rg][c0 + DH * hf] = run;
  }
  if (tid == 0) s.bad = 0;
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
#pragma unroll
    for (int t = 0; t < RPT; ++t) {
      const int n = hf * RPT + t, i = r0 + t;
      gm[n] += offs;
      if ((i & 15) == 0) {
        s.gref[i >> 4][cc] = gm[n];
        s.eref[i >> 4][cc] = __expf(gm[n]);
        s.ecg[i >> 4][cc] = __expf(tot - gm[n]);
      }
      s.u.p.x.Kn[i][cc] = (_Float16)(-kk[n] * __expf(gm[n]));
    }
    if (rg == 0) {
      s.degc[cc] = __expf(tot);   // e^Gam_C until deGC is formed
      s.gcl[cc] = tot;
    }
  }
  if (tid < BC) {
    s.orow[tid] = torow;
    s.irow[tid] = trow;
    s.beta[tid] = tbeta;
  }
#pragma unroll
  for (int n = 0; n < NAV; ++n) {
    const int e = tid + NT * n;
    if (e < BC * BC / 4) *(f16x4*)&s.u.p.A[e / (BC / 4)][(e % (BC / 4)) * 4] = av[n];
  }
  if (tid < BC * 2) *(f16x8*)&s.u.p.Td[tid / 2][(tid % 2) * 8] = tv;
  __syncthreads();
  // gradients in the power-of-two units of the chunk's round (round_scale,
  // stored by the round's reverse pass): dO enters scaled (dy and the
  // end-state gradients come scaled), every gradient leaves times inv.  Read
  // here, behind the prologue's loads and ahead of q's.
  const float sg = __uint_as_float(*scale_word(a.gmax, a.n_rounds, cround));
  const float inv = 1.f / sg;
  const float sc = a.scale * sg;
  {  // decays past the factored range anywhere in the chunk: phase 3 takes exact pairs
    bool bad = steep;
#pragma unroll
    for (int hf = 0; hf < NHF; ++hf)
#pragma unroll
      for (int t = 0; t < RPT; ++t)
        bad |= s.gref[(r0 + t) >> 4][c0 + DH * hf] - gm[hf * RPT + t] > kExactDecay;
    if (bad) s.bad = 1;
  }
  // q (phase 3) through the input rows of the row table: addressed from LDS
  // after the barrier, these loads stay behind the prologue's, whose waits
  // then remain exact
#pragma unroll
  for (int t = 0; t < RPT; ++t) rows[t] = s.irow[r0 + t];
#pragma unroll
  for (int hf = 0; hf < NHF; ++hf)
#pragma unroll
    for (int t = 0; t < RPT; ++t) {
      const int r = rows[t];
      const float w = ld_in(q, ((size_t)(r < 0 ? 0 : r) * H + h) * D + c0 + DH * hf);
      qq[hf * RPT + t] = r >= 0 ? w : 0.f;
    }

  // ---- phase 1: Z = V - (K e^Gam) h on column block `wave` ----
  if (vw) {
    f16x8 hb[KD];
    {
      f32x4 hC[NCB];
#pragma unroll
      for (int C = 0; C < NCB; ++C) {
#pragma unroll
        for (int r = 0; r < 4; ++r) s.u.p.Hs[16 * C + 4 * g + r][col] = hraw[C][r];   // h as [c][v] fp16
        hC[C] = (f32x4){(float)hraw[C][0], (float)hraw[C][1], (float)hraw[C][2], (float)hraw[C][3]};
      }
#pragma unroll
      for (int ks = 0; ks < KD; ++ks) hb[ks] = acc_pair(hC[2 * ks], hC[2 * ks + 1]);
    }
#pragma unroll
    for (int J = 0; J < NB; ++J) z[J] = in4_to_f32(vraw[J]);
#pragma unroll
    for (int J = 0; J < NB; ++J)
#pragma unroll
      for (int ks = 0; ks < KD; ++ks)
        z[J] = mfma16(lds_a_perm(&s.u.p.x.Kn[0][0], G::PD, 16 * J + l16, 32 * ks, g), hb[ks], z[J]);
  }
  __syncthreads();  // Kn is dead: dO takes its place
#pragma unroll
  for (int n = 0; n < NV4; ++n) {
    const int e = tid + NT * n;
    if (e < BC * D / 4) {
      const int t = e >> 6, l = e & 63;   // lane l's piece of tile t: rows i0 .. i0 + 3 of column v
      const int i0 = 16 * (t / (D / 16)) + 4 * (l >> 4), v = 16 * (t % (D / 16)) + (l & 15);
      const f32x4 x = sc * in4_to_f32(dov[n]);
#pragma unroll
      for (int r = 0; r < 4; ++r) s.u.p.x.dO[i0 + r][v] = (_Float16)x[r];
    }
  }
  if (vw) {
#pragma unroll
    for (int J = 0; J < NB; ++J) {
#pragma unroll
      for (int r = 0; r < 4; ++r)   // rows past the chunk hold no gradient
        dyv[J][r] = 16 * J + 4 * g + r < len ? (float)dyh[J][r] : 0.f;
    }
    // delta by block forward substitution with the diagonal inverses
    f32x4 d[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      f32x4 rr = z[I];
#pragma unroll
      for (int J = 0; J < I; ++J) {
        const f16x4 la = *(const f16x4*)&s.u.p.A[16 * I + l16][16 * J + 4 * g];   // -A
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
    float ye[NB][4];  // dy * e
    // e = Z - A delta;  dbeta partial = sum over the columns of dy * e;  dV = beta dy
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      f32x4 e = z[I];
#pragma unroll
      for (int ks = 0; ks < KB; ++ks)
        if (32 * ks <= 16 * I + 15) {
          const f16x8 aa = lds_a_perm(&s.u.p.A[0][0], G::PB, 16 * I + l16, 32 * ks, g, HALF);   // -A
          e = mfma16(aa, db[ks], e);
        }
      float dvv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * g + r;
        const float dy = dyv[I][r], b = s.beta[i];
        ye[I][r] = dy * e[r];
        dvv[r] = inv * (b * dy);
        s.u.p.nZ[i][col] = (_Float16)(-b * dy);
        s.u.p.dl[i][col] = (_Float16)d[I][r];
      }
      // dv as one 16-byte piece of a row per lane
      quad_transpose(dvv);
      const int i = 16 * I + quad_row();
      if (i < len)
        *(float4*)(grad_dst(a, a.dv, a.rep_dv, rep0, s.orow[i], i, nrep, h, D) + col - l16 + quad_col()) =
            make_float4(dvv[0], dvv[1], dvv[2], dvv[3]);
    }
    // dbeta partial over this wave's 16 columns: row 16 I + 4 g + r
    if constexpr (NB == 4) {
      float x[16];
#pragma unroll
      for (int n = 0; n < 16; ++n) x[n] = ye[n / 4][n % 4];
      s.redb[wave][16 * (l16 / 4) + 4 * g + l16 % 4] = row_reduce16x16(x);
    } else {
#pragma unroll
      for (int I = 0; I < NB; ++I)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = row_sum16(ye[I][r]);
          if (l16 == 0) s.redb[wave][16 * I + 4 * g + r] = x;
        }
    }
  }
  __syncthreads();
  if (tid < BC && tid < len) {
    float acc = 0.f;
    for (int w = 0; w < NCB; ++w) acc += s.redb[w][tid];
    *grad_dst(a, a.dbeta, a.rep_db, rep0, s.orow[tid], tid, nrep, h, 1) = inv * acc;
  }
  if (tid < D) {
    for (int I = 0; I < NB; ++I)
      for (int J = 0; J <= I; ++J)
        s.dfac[low_index(I, J)][tid] = __expf(s.gref[I][tid] - s.gref[J][tid]);
  }

  // ---- phase 2: products contracting dv (fp16 matrix cores), transposed tiles ----
  const int tI = wave % NB, tu = wave / NB;
  f32x4 dQt[NTW], dKt[NTW], dKh[NTW];
#pragma unroll
  for (int m = 0; m < NTW; ++m) {
    const int C = tu + NG * m;
    f32x4 x1 = {0.f, 0.f, 0.f, 0.f}, x2 = {0.f, 0.f, 0.f, 0.f};
    if (C < NCB) {
#pragma unroll
      for (int ks = 0; ks < KD; ++ks) {
        const f16x8 ah = *(const f16x8*)&s.u.p.Hs[16 * C + l16][32 * ks + 8 * g];
        x1 = mfma16(ah, *(const f16x8*)&s.u.p.x.dO[16 * tI + l16][32 * ks + 8 * g], x1);
        x2 = mfma16(ah, *(const f16x8*)&s.u.p.nZ[16 * tI + l16][32 * ks + 8 * g], x2);
      }
    }
    dQt[m] = x1;
    dKt[m] = x2;
  }
  // dP / dA blocks met by row block tI: slot sl <= tI is (tI, J = sl) as a [j][i]
  // tile, slot sl > tI is (I = sl - 1, tI) as an [i][j] tile
  s16x4 Ph[NS], Pl[NS], Ah[NS], Al[NS];
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) {
    const bool rside = sl <= tI;
    const _Float16* a1 = rside ? &s.u.p.dl[16 * sl][0] : &s.u.p.x.dO[16 * (sl - 1)][0];
    const _Float16* a2 = rside ? &s.u.p.dl[16 * sl][0] : &s.u.p.nZ[16 * (sl - 1)][0];
    const _Float16* b1 = rside ? &s.u.p.x.dO[16 * tI][0] : &s.u.p.dl[16 * tI][0];
    const _Float16* b2 = rside ? &s.u.p.nZ[16 * tI][0] : &s.u.p.dl[16 * tI][0];
    f32x4 tp = {0.f, 0.f, 0.f, 0.f}, ta = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KD; ++ks) {
      const int o = l16 * G::PD + 32 * ks + 8 * g;
      tp = mfma16(*(const f16x8*)(a1 + o), *(const f16x8*)(b1 + o), tp);
      ta = mfma16(*(const f16x8*)(a2 + o), *(const f16x8*)(b2 + o), ta);
    }
    // diagonal blocks: keep j <= i (P) and j < i (A)
    const bool diag = rside ? (sl == tI) : (sl == tI + 1);
    if (diag) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rw = 4 * g + r;            // tile row
        const int jj = rside ? rw : l16;     // j within the block
        const int ii = rside ? l16 : rw;     // i within the block
        if (jj > ii) tp[r] = 0.f;
        if (jj >= ii) ta[r] = 0.f;
      }
    }
    split_tile(tp, Ph[sl], Pl[sl]);
    split_tile(ta, Ah[sl], Al[sl]);
  }
  if (vw) {
    // deGC partial over this wave's 16 columns: channel 16 C + 4 g + r, the
    // sum over v of h dh' (h as its fp16 copy, which holds exactly the stored
    // start state); the 16 lanes of a row group hold the 16 columns, summed
    // by row_reduce16x16 (lane l16 ends with the sum of value l16)
    static_assert(NCB == 4 || NCB == 8, "head dim 64 or 128");
    float x0[16], x1[16];
#pragma unroll
    for (int C = 0; C < NCB; ++C)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = (float)hraw[C][r] * (float)dhraw[C][r];
        if (C < 4) x0[4 * C + r] = p; else x1[4 * (C - 4) + r] = p;
      }
    s.redg[wave][16 * (l16 >> 2) + 4 * g + (l16 & 3)] = row_reduce16x16(x0);
    if constexpr (NCB == 8) s.redg[wave][16 * (4 + (l16 >> 2)) + 4 * g + (l16 & 3)] = row_reduce16x16(x1);
  }
  __syncthreads();  // h is dead: dh' takes its place
  if (vw) {
#pragma unroll
    for (int C = 0; C < NCB; ++C)
#pragma unroll
      for (int r = 0; r < 4; ++r) s.u.p.Hs[16 * C + 4 * g + r][col] = dhraw[C][r];
  }
  if (tid < D) {
    float acc = 0.f;
    for (int w = 0; w < NCB; ++w) acc += s.redg[w][tid];
    s.degc[tid] *= acc;   // deGC e^Gam_C
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < NTW; ++m) {
    const int C = tu + NG * m;
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (C < NCB) {
#pragma unroll
      for (int ks = 0; ks < KD; ++ks)
        x = mfma16(*(const f16x8*)&s.u.p.Hs[16 * C + l16][32 * ks + 8 * g],
                   *(const f16x8*)&s.u.p.dl[16 * tI + l16][32 * ks + 8 * g], x);
    }
    dKh[m] = x;
  }

  // ---- phase 3: decay-weighted products and the combine, 64 channels per pass ----
  const bool exact = s.bad != 0;   // block-uniform (set before two barriers)
#pragma unroll
  for (int hf = 0; hf < NHF; ++hf) {
    __syncthreads();  // the previous phase's LDS readers are done
    if (exact) {
      phase3_exact_stage<BC, D>(s, hf, gm, qq, kk, Ph, Pl, Ah, Al, tI, tu);
    } else {  // staging: channel c0 of the pass, rows r0 .. r0 + RPT - 1
      const int ch = DH * hf + c0;
      if constexpr (RPT == 8) {   // the thread's 8 rows are one 16-byte run of each [c][i] array
        bf16x8 rh8, rl8, qh8, ql8, kh8, kl8;
        float rv[8], qv[8], kv[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int n = hf * RPT + t, i = r0 + t;
          const float ref = s.gref[i >> 4][ch];
          const float f = __expf(gm[n] - ref), fi = __expf(ref - gm[n]);
          rv[t] = kk[n] * fi;
          qv[t] = qq[n] * f;
          kv[t] = kk[n] * f;
          s.u.d.gam[c0][i] = gm[n];
        }
        split8(rv, rh8, rl8);
        split8(qv, qh8, ql8);
        split8(kv, kh8, kl8);
        put8(&s.u.d.rh[c0][r0], rh8); put8(&s.u.d.rl[c0][r0], rl8);
        put8(&s.u.d.qh[c0][r0], qh8); put8(&s.u.d.ql[c0][r0], ql8);
        put8(&s.u.d.kh[c0][r0], kh8); put8(&s.u.d.kl[c0][r0], kl8);
        if constexpr (RAWQK) {
          bf16x8 q8, k8;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            q8[t] = (__bf16)qq[hf * RPT + t];
            k8[t] = (__bf16)kk[hf * RPT + t];
          }
          put8(&s.u.d.qraw[c0][r0], q8);
          put8(&s.u.d.kraw[c0][r0], k8);
        }
      } else {
#pragma unroll
        for (int t = 0; t < RPT; ++t) {
          const int n = hf * RPT + t, i = r0 + t;
          const float ref = s.gref[i >> 4][ch];
          const float f = __expf(gm[n] - ref), fi = __expf(ref - gm[n]);
          __bf16 x, y;
          split_bf16(kk[n] * fi, x, y);
          s.u.d.rh[c0][i] = x; s.u.d.rl[c0][i] = y;
          split_bf16(qq[n] * f, x, y);
          s.u.d.qh[c0][i] = x; s.u.d.ql[c0][i] = y;
          split_bf16(kk[n] * f, x, y);
          s.u.d.kh[c0][i] = x; s.u.d.kl[c0][i] = y;
          s.u.d.gam[c0][i] = gm[n];
          if constexpr (RAWQK) {
            s.u.d.qraw[c0][i] = (__bf16)qq[n];
            s.u.d.kraw[c0][i] = (__bf16)kk[n];
          }
        }
      }
    }
    __syncthreads();
    if (exact) {
#pragma unroll
      for (int m = 0; m < NTW; ++m) {
        const int C = tu + NG * m;
        if (C < NCB && C / 4 == hf)
          phase3_exact_tile<BC, D>(a, s, hf, C, tI, dQt[m], dKt[m], dKh[m], rep0, nrep, len, h,
                                   inv);
      }
    } else {
#pragma unroll
    for (int m = 0; m < NTW; ++m) {
      const int C = tu + NG * m;
      if (C < NCB && C / 4 == hf) {
        const int cb = 16 * (C % 4);          // first channel of the tile within the pass
        const int ca = cb + l16;              // A-operand row (channel) of this lane
        const int cf = DH * hf + cb + 4 * g;  // first output channel of this lane
        f32x4 rP = {0.f, 0.f, 0.f, 0.f}, rA = rP, cP = rP, cA = rP;
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
          if (sl <= tI) {  // row side, block pair (tI, J = sl), around gref_J
            const int J = sl;
            const s16x4 ah = *(const s16x4*)&s.u.d.rh[ca][16 * J + 4 * g];
            const s16x4 al = *(const s16x4*)&s.u.d.rl[ca][16 * J + 4 * g];
            const f32x4 tp = mma3(ah, al, Ph[sl], Pl[sl]);
            const f32x4 ta = mma3(ah, al, Ah[sl], Al[sl]);
            const float4 f = *(const float4*)&s.dfac[low_index(tI, J)][cf];
            rP[0] += f.x * tp[0]; rP[1] += f.y * tp[1]; rP[2] += f.z * tp[2]; rP[3] += f.w * tp[3];
            rA[0] += f.x * ta[0]; rA[1] += f.y * ta[1]; rA[2] += f.z * ta[2]; rA[3] += f.w * ta[3];
          } else {         // column side, block pair (I = sl - 1, tI), around gref_tI
            const int I = sl - 1;
            const s16x4 qh = *(const s16x4*)&s.u.d.qh[ca][16 * I + 4 * g];
            const s16x4 ql = *(const s16x4*)&s.u.d.ql[ca][16 * I + 4 * g];
            const s16x4 kh = *(const s16x4*)&s.u.d.kh[ca][16 * I + 4 * g];
            const s16x4 kl = *(const s16x4*)&s.u.d.kl[ca][16 * I + 4 * g];
            const f32x4 tp = mma3(qh, ql, Ph[sl], Pl[sl]);
            const f32x4 ta = mma3(kh, kl, Ah[sl], Al[sl]);
            const float4 f = *(const float4*)&s.dfac[low_index(I, tI)][cf];
            cP[0] += f.x * tp[0]; cP[1] += f.y * tp[1]; cP[2] += f.z * tp[2]; cP[3] += f.w * tp[3];
            cA[0] += f.x * ta[0]; cA[1] += f.y * ta[1]; cA[2] += f.z * ta[2]; cA[3] += f.w * ta[3];
          }
        }
        // combine: lane element (channel cf + r, row i)
        const int i = 16 * tI + l16;
        float4 vq, vk;
        float cs[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int cl = cb + 4 * g + r, ch = cf + r;
          const float gam = s.u.d.gam[cl][i];
          const float ref = s.gref[tI][ch], er = s.eref[tI][ch], eg = s.ecg[tI][ch];
          const float lf = __expf(gam - ref), rf = __expf(ref - gam);
          float qd, kd, kr;   // q e^(Gam-ref), k e^(Gam-ref), k e^(ref-Gam)
          if constexpr (RAWQK) {
            const float qv = bf16_val(s.u.d.qraw[cl][i]), kv = bf16_val(s.u.d.kraw[cl][i]);
            qd = qv * lf;
            kd = kv * lf;
            kr = kv * rf;
          } else {
            qd = bf16_val(s.u.d.qh[cl][i]) + bf16_val(s.u.d.ql[cl][i]);
            kd = bf16_val(s.u.d.kh[cl][i]) + bf16_val(s.u.d.kl[cl][i]);
            kr = bf16_val(s.u.d.rh[cl][i]) + bf16_val(s.u.d.rl[cl][i]);
          }
          const float xq = dQt[m][r] * er + rP[r];
          const float xk = dKt[m][r] * er + rA[r];
          const float kh2 = dKh[m][r] * kr * eg;
          cs[r] = kh2;
          s.u.d.gam[cl][i] = xq * qd + xk * kd - kh2 - kr * (cP[r] + cA[r]);   // dGam, this lane's
          (&vq.x)[r] = xq * lf;
          (&vk.x)[r] = xk * lf + (dKh[m][r] * eg + cP[r] + cA[r]) * rf;
        }
        if (i < len) {
          const int orow = s.orow[i];
          *(float4*)(grad_dst(a, a.dq, a.rep_dq, rep0, orow, i, nrep, h, D) + cf) =
              make_float4(inv * vq.x, inv * vq.y, inv * vq.z, inv * vq.w);
          *(float4*)(grad_dst(a, a.dk, a.rep_dk, rep0, orow, i, nrep, h, D) + cf) =
              make_float4(inv * vk.x, inv * vk.y, inv * vk.z, inv * vk.w);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = row_sum16(cs[r]);
          if (l16 == 0) s.csum[tI][cf + r] = x;
        }
      }
    }
    }
    __syncthreads();
    // dg = reverse cumulative sum of dGam, the Gam_C terms entering at the last row
    const int ch = DH * hf + c0;
    const float* dgr = exact ? &s.u.e.dgam[c0][0] : &s.u.d.gam[c0][0];
    float loc[RPT];
    float run = 0.f;
#pragma unroll
    for (int t = RPT - 1; t >= 0; --t) {
      run += dgr[r0 + t];
      loc[t] = run;
    }
    s.part[rg][ch] = run;
    __syncthreads();
    float tail = s.degc[ch];
#pragma unroll
    for (int I = 0; I < NB; ++I) tail += s.csum[I][ch];
#pragma unroll
    for (int j = 0; j < NRG; ++j) tail += (j > rg) ? s.part[j][ch] : 0.f;
#pragma unroll
    for (int t = 0; t < RPT; ++t) {
      const int i = r0 + t;
      if (i < len) grad_dst(a, a.dg, a.rep_dg, rep0, s.orow[i], i, nrep, h, D)[ch] = inv * (loc[t] + tail);
    }
  }
}

template <typename TIn, int BC, int D>
hipError_t launch_grad_t(const BwdArgs& a, int c_begin, int n_chunks, hipStream_t st) {
  if (n_chunks <= 0) return hipSuccess;
  KDA_LAUNCH("kda_bwd_chunk_grad", (k_bwd_grad<TIn, BC, D>), dim3(n_chunks, a.H), dim3(NT), st, a,
             c_begin);
  return hipGetLastError();
}

// chunks c_begin .. c_begin + n_chunks - 1
hipError_t launch_grad(const BwdArgs& a, bool bf16, int BC, int D, int c_begin, int n_chunks,
                       hipStream_t st) {
#define KDA_GRAD_CASE(T, BCv, Dv) \
  if (BC == BCv && D == Dv) return launch_grad_t<T, BCv, Dv>(a, c_begin, n_chunks, st);
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
