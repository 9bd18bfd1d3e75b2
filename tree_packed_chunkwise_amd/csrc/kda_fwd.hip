// kda_fwd.hip -- fused forward of one packed round (gfx950).
//
// One block per (sequence, head, dv slice) of the round (HARTS Figure 2(c):
// all sequences of a round form one packed call).  The block walks its
// sequence's chunks in order; per chunk (C rows, state h of dk x dv) it
// copies the chunk's forward image (written by the chunk-parallel pass,
// kda_prep.hip: q e^Gam, -k e^Gam, (k e^(Gam_C - Gam))^T, A, P, the
// diagonal-block inverses Td, e^Gam_C, beta, V) into LDS and runs:
//   Z     = V - (K e^Gam) h                 (value minus the decayed state's prediction)
//   delta : (I + diag(beta) A) delta = diag(beta) Z   (the delta-rule writes of
//                                            the chunk's rows; block substitution)
//   O     = scale ((Q e^Gam) h + P delta)   (written for non-replay rows only, Figure C.1(b))
//   h'    = diag(e^Gam_C) h + (K e^(Gam_C - Gam))^T delta
// The state h and the chunk's Z / delta never leave registers: they are MFMA
// accumulators reused as B operands (chunk.h).  The next chunk's image is
// copied asynchronously into a second LDS buffer (and its V into registers)
// while the current chunk's state phase runs, so the sequential chain waits
// on no global load.  The start state of every chunk
// is saved for the reverse pass; handoff states are saved at chunk ends; the
// leaf state is written at the end of the sequence.
//
// dv slicing: a block owns NV 16-wide column blocks of the state (one per
// wave); a round with few sequences is cut into D/(16 NV) slices so that more
// compute units work on it.
#include "chunk.h"
#include "timing.h"

namespace kda {

template <typename TIn, int BC, int D, int NV>
__global__ __launch_bounds__(NT) void k_fwd_round(FwdArgs a, int seq_begin) {
  using G = Geom<BC, D>;
  using FH = FwdHead<BC, D>;
  using FI = FwdImage<BC, D, TIn>;
  static_assert(NV <= NW, "one column block per wave");
  constexpr int KD = D / 32;                 // 32-deep k steps over the head dim
  constexpr int KB = (BC + 31) / 32;         // 32-deep k steps over the chunk rows
  constexpr bool HALF = (BC == 16);          // chunk rows cover half a k step
  constexpr int NVEC = (int)(sizeof(FH) / 16);
  __shared__ FH buf[2];                      // this chunk's image and the next one's
  // blocks in the round's launch order: sequence rank major, head minor
  const int seq = ld_uni(a.plan.seq_lpt, seq_begin + (int)blockIdx.x / a.H);
  const int h = (int)blockIdx.x % a.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const bool sw = wave < NV;                 // this wave carries a column block of the state
  const int col = 16 * (blockIdx.z * NV + wave) + l16;
  const int cq = col - l16 + quad_col();     // first column of this lane's row piece
  const int rq = quad_row();                 // its row within a 16-row block
  const int H = a.H;
  const size_t DD = (size_t)D * D;
  const int cbeg = ld_uni(a.plan.seq_chunk_ptr, seq);
  const int cend = ld_uni(a.plan.seq_chunk_ptr, seq + 1);
  auto image = [&](int cc) { return a.fimg + ((size_t)cc * H + h) * fwd_image_bytes(BC, D); };

  f32x4 hs[G::NCB];
  {
    const float* src = nullptr;
    if (ld_uni(a.plan.seq_init_kind, seq) == 0) {
      if (a.h0) src = a.h0 + ((size_t)ld_uni(a.plan.seq_init_idx, seq) * H + h) * DD;
    } else {
      src = a.bufs + ((size_t)ld_uni(a.plan.seq_init_idx, seq) * H + h) * DD;
    }
#pragma unroll
    for (int C = 0; C < G::NCB; ++C)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        hs[C][r] = (src && sw) ? src[(size_t)(16 * C + 4 * g + r) * D + col] : 0.f;
  }
  // V of the chunk in flight, raw: this lane's accumulator piece of every
  // 16-row block (one vector load each from the image's V tiles)
  in4_t<TIn> vr[G::NB];
  auto load_v = [&](int cc) {
    const FI* F = (const FI*)image(cc);
#pragma unroll
    for (int J = 0; J < G::NB; ++J)
      vr[J] = sw ? *(const in4_t<TIn>*)(&F->V[0][0] + state_tile<D>(J, col >> 4)) : (in4_t<TIn>)0;
  };
  if (cbeg < cend) {
    lds_copy_async_untracked(&buf[0], image(cbeg), NVEC);
    load_v(cbeg);
  }
  for (int c = cbeg; c < cend; ++c) {
    const size_t blk = (size_t)c * H + h;
    __builtin_amdgcn_s_waitcnt(0);  // this chunk's image (and V) have landed ...
    __syncthreads();                // ... for every wave; the other buffer is free
    const FH& s = buf[(c - cbeg) & 1];
    f32x4 z[G::NB];
#pragma unroll
    for (int J = 0; J < G::NB; ++J) z[J] = in4_to_f32(vr[J]);
    // the next chunk's image, in two parts: the second once this wave's
    // first products are issued
    if (c + 1 < cend) lds_copy_async_untracked<2>(&buf[(c - cbeg + 1) & 1], image(c + 1), NVEC, 0);
    if (!sw && c + 1 < cend) lds_copy_async_untracked<2>(&buf[(c - cbeg + 1) & 1], image(c + 1), NVEC, 1);

    // ---- state phase: wave w < NV owns column block w of the slice ----
    if (sw) {
      const float sc = a.scale;
      {  // start state of the chunk, kept for the reverse pass (fp16: its only
         // consumers feed it to fp16 matrix cores)
        _Float16* dst = a.chunk_h + blk * DD;
#pragma unroll
        for (int C = 0; C < G::NCB; ++C) st_h4(dst + state_tile<D>(C, col >> 4), hs[C]);
      }
      f16x8 hb[KD];
#pragma unroll
      for (int ks = 0; ks < KD; ++ks) hb[ks] = acc_pair(hs[2 * ks], hs[2 * ks + 1]);
      // Every phase first issues all of its LDS fragment reads, then its
      // MFMAs, so that the reads are in flight together.
      // Z = V - (K e^Gam) h
      f16x8 fa[G::NB][KD];
#pragma unroll
      for (int J = 0; J < G::NB; ++J)
#pragma unroll
        for (int ks = 0; ks < KD; ++ks) fa[J][ks] = lds_a_perm_sw<D>(&s.Kn[0][0], 16 * J + l16, 32 * ks, g);
      __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the products
#pragma unroll
      for (int J = 0; J < G::NB; ++J)
#pragma unroll
        for (int ks = 0; ks < KD; ++ks) z[J] = mfma16(fa[J][ks], hb[ks], z[J]);
      // the next chunk's V, into the registers this chunk's V has left
      // (loaded on every step, so that they stay the same registers)
      load_v(c + 1 < cend ? c + 1 : c);
      if (c + 1 < cend) lds_copy_async_untracked<2>(&buf[(c - cbeg + 1) & 1], image(c + 1), NVEC, 1);
      // (Q e^Gam) h: independent of the solve below, so it overlaps it
#pragma unroll
      for (int I = 0; I < G::NB; ++I)
#pragma unroll
        for (int ks = 0; ks < KD; ++ks) fa[I][ks] = lds_a_perm_sw<D>(&s.Qt[0][0], 16 * I + l16, 32 * ks, g);
      __builtin_amdgcn_sched_barrier(0);
      f32x4 o[G::NB];
#pragma unroll
      for (int I = 0; I < G::NB; ++I) {
        o[I] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KD; ++ks) o[I] = mfma16(fa[I][ks], hb[ks], o[I]);
      }
      // (I + diag(beta) A) delta = diag(beta) Z, block forward substitution with
      // the diagonal inverses: delta_I = Td_I diag(beta_I) (Z_I - sum_{J<I} A_IJ delta_J)
      f16x4 fl[G::NB][G::NB], ft[G::NB];
#pragma unroll
      for (int I = 0; I < G::NB; ++I) {
        ft[I] = *(const f16x4*)&s.Td[16 * I + l16][4 * g];
#pragma unroll
        for (int J = 0; J < I; ++J)   // columns 16 J + 4 g .. of the swizzled row
          fl[I][J] = *(const f16x4*)&s.L[16 * I + l16][4 * swz_piece<BC>(4 * J, g ^ swz_term<BC>(l16))];
      }
      f32x4 bz[G::NB];
#pragma unroll
      for (int I = 0; I < G::NB; ++I)
#pragma unroll
        for (int r = 0; r < 4; ++r) bz[I][r] = s.beta[16 * I + 4 * g + r];
      __builtin_amdgcn_sched_barrier(0);
      f32x4 d[G::NB];
#pragma unroll
      for (int I = 0; I < G::NB; ++I) {
        f32x4 rr = z[I];
#pragma unroll
        for (int J = 0; J < I; ++J) rr = mfma16k16(fl[I][J], acc4(d[J]), rr);
        rr *= bz[I];
        d[I] = mfma16k16(ft[I], acc4(rr), (f32x4){0.f, 0.f, 0.f, 0.f});
      }
      f16x8 db[KB];
#pragma unroll
      for (int ks = 0; ks < KB; ++ks) db[ks] = HALF ? acc_half(d[0]) : acc_pair(d[2 * ks], d[2 * ks + 1]);
      // O = scale ((Q e^Gam) h + P delta)
      f16x8 fp[G::NB][KB];
#pragma unroll
      for (int I = 0; I < G::NB; ++I)
#pragma unroll
        for (int ks = 0; ks < KB; ++ks)
          if (32 * ks <= 16 * I + 15) fp[I][ks] = lds_a_perm_sw<BC>(&s.P[0][0], 16 * I + l16, 32 * ks, g, HALF);
      // (K e^(Gam_C-Gam))^T fragments for the state update
      f16x8 fk[G::NCB][KB];
#pragma unroll
      for (int C = 0; C < G::NCB; ++C)
#pragma unroll
        for (int ks = 0; ks < KB; ++ks) fk[C][ks] = lds_a_perm_sw<BC>(&s.KhT[0][0], 16 * C + l16, 32 * ks, g, HALF);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int I = 0; I < G::NB; ++I) {
#pragma unroll
        for (int ks = 0; ks < KB; ++ks)
          if (32 * ks <= 16 * I + 15) o[I] = mfma16(fp[I][ks], db[ks], o[I]);
        o[I] *= sc;
        quad_transpose(o[I]);
        const int orow = s.orow[16 * I + rq];
        if (orow >= 0) *(f32x4*)&a.o[((size_t)orow * H + h) * D + cq] = o[I];
      }
      // h' = diag(e^Gam_C) h + (K e^(Gam_C-Gam))^T delta
#pragma unroll
      for (int C = 0; C < G::NCB; ++C) {
#pragma unroll
        for (int r = 0; r < 4; ++r) hs[C][r] *= s.gc[16 * C + 4 * g + r];
#pragma unroll
        for (int ks = 0; ks < KB; ++ks) hs[C] = mfma16(fk[C][ks], db[ks], hs[C]);
      }
      const int save = ld_uni(a.plan.chunk_save, c);
      if (save >= 0) {
        float* dst = a.bufs + ((size_t)save * H + h) * DD;
#pragma unroll
        for (int C = 0; C < G::NCB; ++C)
#pragma unroll
          for (int r = 0; r < 4; ++r) dst[(size_t)(16 * C + 4 * g + r) * D + col] = hs[C][r];
      }
    }
  }
  if (sw && ld_uni(a.plan.seq_leaf, seq) >= 0) {   // node-wise sequences may end at an inner segment
    float* dst = a.h_leaf + ((size_t)ld_uni(a.plan.seq_leaf, seq) * H + h) * DD;
#pragma unroll
    for (int C = 0; C < G::NCB; ++C)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(size_t)(16 * C + 4 * g + r) * D + col] = hs[C][r];
  }
}

// Slices of a round: as many as keep every block on its own compute unit
// (256 CUs) without exceeding D/16 column blocks or max_slices (<= 0: no
// limit of its own).  A round that runs beside prep or gradient work on a
// second stream takes fewer: its chain is bound by each block's own
// bandwidth, so the compute units it leaves go to the throughput kernels.
int round_slices(int nseq, int H, int D, int max_slices) {
  const int maxs = max_slices > 0 && max_slices < D / 16 ? max_slices : D / 16;
  int sl = 1;
  while (sl * 2 <= maxs && (long)nseq * H * sl * 2 <= 256) sl *= 2;
  return sl;
}

template <typename TIn, int BC, int D, int NV>
hipError_t launch_round(const FwdArgs& a, int nseq, int seq0, int slices, hipStream_t st) {
  KDA_LAUNCH("kda_fwd_round", (k_fwd_round<TIn, BC, D, NV>), dim3(nseq * a.H, 1, slices), dim3(NT),
             st, a, seq0);
  return hipGetLastError();
}

template <typename TIn, int BC, int D>
hipError_t launch_fwd2_t(const FwdArgs& a, const int* round_ptr_host, int r_begin, int r_end,
                         int max_slices, hipStream_t st) {
  constexpr int NCB = D / 16;
  for (int r = r_begin; r < r_end; ++r) {
    const int nseq = round_ptr_host[r + 1] - round_ptr_host[r];
    if (nseq == 0) continue;
    const int sl = round_slices(nseq, a.H, D, max_slices);
    const int nv = NCB / sl;
    hipError_t e = hipErrorInvalidValue;
    if (nv == NCB) e = launch_round<TIn, BC, D, NCB>(a, nseq, round_ptr_host[r], sl, st);
    else if (nv == 4) e = launch_round<TIn, BC, D, 4>(a, nseq, round_ptr_host[r], sl, st);
    else if (nv == 2) e = launch_round<TIn, BC, D, 2>(a, nseq, round_ptr_host[r], sl, st);
    else if (nv == 1) e = launch_round<TIn, BC, D, 1>(a, nseq, round_ptr_host[r], sl, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// rounds r_begin .. r_end - 1, in order
hipError_t launch_fwd_rounds(const FwdArgs& a, bool bf16, int BC, int D, const int* round_ptr_host,
                             int r_begin, int r_end, int max_slices, hipStream_t st) {
#define KDA_FWD_CASE(T, BCv, Dv) \
  if (BC == BCv && D == Dv) return launch_fwd2_t<T, BCv, Dv>(a, round_ptr_host, r_begin, r_end, max_slices, st);
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
