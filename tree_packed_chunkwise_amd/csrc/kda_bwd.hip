// kda_bwd.hip -- reverse pass of one packed round: the state-gradient
// recurrence (gfx950).
//
// One block per (sequence, head, dv slice) of the round, rounds in reverse
// order; the block walks its sequence's chunks backwards carrying dh, the
// gradient of the state at the current chunk end (it starts from the leaf
// state's gradient).  Per chunk it copies the head of the chunk's forward
// image (written by the chunk-parallel pass, kda_prep.hip: q e^Gam,
// -k e^Gam, (k e^(Gam_C - Gam))^T, A, P, Td, e^Gam_C, beta) into LDS; each
// transposed operand below is read from it with the transposing LDS read
// (lds_a_perm_tr / lds_tr4 in chunk.h), and the scale is folded into dO.
// Then:
//   at a handoff chunk end: dh += start gradients of every sequence that
//        started from that state (later rounds, already final); the total is
//        the handoff state's gradient (HARTS abstract: differentiable
//        boundary-state handoff)
//   ddelta = scale P^T dO + (K e^(Gam_C - Gam)) dh          (dO = 0 on replay rows)
//   dy     : (I + diag(beta) A)^T dy = ddelta                (block back substitution)
//   dh     <- diag(e^Gam_C) dh + scale (Q e^Gam)^T dO - (K e^Gam)^T diag(beta) dy
// and writes dy and the chunk-end dh for the chunk-local gradient pass; the
// sequence's start gradient goes to its slot.  dh, ddelta and dy stay in
// registers (MFMA accumulators reused as B operands, see chunk.h).  The
// previous chunk's image is copied asynchronously into a second LDS buffer
// (and its dO rows into registers) while the current chunk's state phase
// runs.  Each round runs in the power-of-two units of round_scale (common.h).
#include "chunk.h"
#include "timing.h"

namespace kda {

__device__ inline float in_f32(float x) { return x; }
__device__ inline float in_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

template <typename TIn, int BC, int D, int NV>
__global__ __launch_bounds__(NT) void k_bwd_round(BwdArgs a, int seq_begin, int round) {
  using G = Geom<BC, D>;
  using BI = FwdHead<BC, D>;
  static_assert(NV <= NW, "one column block per wave");
  constexpr int KD = D / 32;
  constexpr int KB = (BC + 31) / 32;
  constexpr bool HALF = (BC == 16);
  constexpr int NVEC = (int)(sizeof(BI) / 16);
  __shared__ BI buf[2];   // this chunk's image and the next one's (chunks run backwards)
  // blocks in the round's launch order: sequence rank major, head minor
  const int seq = ld_uni(a.plan.seq_lpt, seq_begin + (int)blockIdx.x / a.H);
  const int h = (int)blockIdx.x % a.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const bool sw = wave < NV;
  const int col = 16 * (blockIdx.z * NV + wave) + l16;
  const int H = a.H;
  const TIn* dOp = (const TIn*)a.dOp;
  const size_t DD = (size_t)D * D;
  const int cbeg = ld_uni(a.plan.seq_chunk_ptr, seq);
  const int cend = ld_uni(a.plan.seq_chunk_ptr, seq + 1);
  auto image = [&](int cc) { return a.fimg + ((size_t)cc * H + h) * fwd_image_bytes(BC, D); };

  f32x4 dh[G::NCB];
  {
    const int leaf = ld_uni(a.plan.seq_leaf, seq);   // -1: the sequence ends at an inner segment
    const float* src = (a.dh_leaf && leaf >= 0) ? a.dh_leaf + ((size_t)leaf * H + h) * DD : nullptr;
#pragma unroll
    for (int C = 0; C < G::NCB; ++C)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        dh[C][r] = (src && sw) ? src[(size_t)(16 * C + 4 * g + r) * D + col] : 0.f;
  }
  // dO of the chunk in flight, raw: this lane's accumulator piece of the
  // 16-row halves of every 32-deep k step, from the chunk's dO tiles (zero on
  // replay rows and past the chunk); two of them form a B fragment
  in4_t<TIn> dor[KB][2];
  auto load_do = [&](int cc) {
    const TIn* src = dOp + ((size_t)cc * H + h) * (BC * D);
#pragma unroll
    for (int ks = 0; ks < KB; ++ks)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        dor[ks][hf] = (in4_t<TIn>)0;
        if (sw && 32 * ks + 16 * hf < BC)
          dor[ks][hf] = *(const in4_t<TIn>*)&src[state_tile<D>(2 * ks + hf, col >> 4)];
      }
  };
  if (cbeg < cend) {
    lds_copy_async_untracked(&buf[0], image(cend - 1), NVEC);
    load_do(cend - 1);
  }
  // the round's gradients in units scaled by sg (round_scale, common.h): dO,
  // dh_leaf and later rounds' start-state gradients enter scaled, the
  // handoff-state and start-state gradients leave unscaled; dy and the
  // chunk-end dh stay scaled for the chunk-local pass (which reads sg back).
  // Its words are read behind the first chunk's loads.
  float later = 0.f;
  const float sg = round_scale(a.gmax, a.n_rounds, round, a.scale, &later), inv = 1.f / sg;
  const float dscale = a.scale * sg;
  if (blockIdx.x == 0 && blockIdx.z == 0 && tid == 0) {
    *suffix_word(a.gmax, a.n_rounds, round) = __float_as_uint(later);
    *scale_word(a.gmax, a.n_rounds, round) = __float_as_uint(sg);
  }
#pragma unroll
  for (int C = 0; C < G::NCB; ++C) dh[C] *= sg;
  for (int c = cend - 1; c >= cbeg; --c) {
    const int len = ld_uni(a.plan.chunk_len, c);
    const size_t blk = (size_t)c * H + h;
    __builtin_amdgcn_s_waitcnt(0);  // this chunk's image (and dO) have landed ...
    __syncthreads();                // ... for every wave; the other buffer is free
    const BI& s = buf[(cend - 1 - c) & 1];
    f32x4 dof[KB][2];
#pragma unroll
    for (int ks = 0; ks < KB; ++ks)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) dof[ks][hf] = dscale * in4_to_f32(dor[ks][hf]);
    if (c > cbeg) {
      lds_copy_async_untracked(&buf[(cend - c) & 1], image(c - 1), NVEC);
      load_do(c - 1);
    }

    if (sw) {
      f16x8 dob[KB];
#pragma unroll
      for (int ks = 0; ks < KB; ++ks) dob[ks] = acc_pair(dof[ks][0], dof[ks][1]);
      const int save = ld_uni(a.plan.chunk_save, c);
      if (save >= 0) {
        const int p0 = ld_uni(a.plan.buf_cons_ptr, save), p1 = ld_uni(a.plan.buf_cons_ptr, save + 1);
        for (int pi = p0; pi < p1; ++pi) {
          const float* src = a.slot + ((size_t)ld_uni(a.plan.buf_cons, pi) * H + h) * DD;
#pragma unroll
          for (int C = 0; C < G::NCB; ++C)
#pragma unroll
            for (int r = 0; r < 4; ++r) dh[C][r] += sg * src[(size_t)(16 * C + 4 * g + r) * D + col];
        }
        if (a.dh_boundary) {
          float* dst = a.dh_boundary + ((size_t)save * H + h) * DD;
#pragma unroll
          for (int C = 0; C < G::NCB; ++C)
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(size_t)(16 * C + 4 * g + r) * D + col] = inv * dh[C][r];
        }
      }
      {
        _Float16* dst = a.dhc + blk * DD;  // fp16 copy for the chunk-local pass
#pragma unroll
        for (int C = 0; C < G::NCB; ++C) st_h4(dst + state_tile<D>(C, col >> 4), dh[C]);
      }
      f16x8 dhb[KD];
#pragma unroll
      for (int ks = 0; ks < KD; ++ks) dhb[ks] = acc_pair(dh[2 * ks], dh[2 * ks + 1]);
      // Every phase first issues its LDS fragment reads, then its MFMAs, so
      // that the reads are in flight together; the three largest phases run
      // as two batches of eight fragments each, which keeps the kernel
      // within its registers.
      // ddelta = scale P^T dO + (K e^(Gam_C-Gam)) dh
      constexpr int HB = G::NB > 1 ? G::NB / 2 : 1;   // row blocks per batch
      constexpr int HC = G::NCB / 2;                  // column blocks per batch
      f32x4 dd[G::NB];
#pragma unroll
      for (int J0 = 0; J0 < G::NB; J0 += HB) {
        f16x8 fb[HB][KD];
#pragma unroll
        for (int j = 0; j < HB; ++j)
#pragma unroll
          for (int ks = 0; ks < KD; ++ks) fb[j][ks] = lds_a_perm_tr_sw<BC>(&s.KhT[0][0], 32 * ks, 16 * (J0 + j));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < HB; ++j) {
          dd[J0 + j] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KD; ++ks) dd[J0 + j] = mfma16(fb[j][ks], dhb[ks], dd[J0 + j]);
        }
      }
      // dh <- diag(e^Gam_C) dh + scale (Q e^Gam)^T dO (dhb holds the old dh)
#pragma unroll
      for (int C0 = 0; C0 < G::NCB; C0 += HC) {
        f16x8 fb[HC][KB];
        f32x4 gcv[HC];
#pragma unroll
        for (int c = 0; c < HC; ++c) {
#pragma unroll
          for (int ks = 0; ks < KB; ++ks) fb[c][ks] = lds_a_perm_tr_sw<D>(&s.Qt[0][0], 32 * ks, 16 * (C0 + c), HALF);
#pragma unroll
          for (int r = 0; r < 4; ++r) gcv[c][r] = s.gc[16 * (C0 + c) + 4 * g + r];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < HC; ++c) {
          dh[C0 + c] *= gcv[c];
#pragma unroll
          for (int ks = 0; ks < KB; ++ks) dh[C0 + c] = mfma16(fb[c][ks], dob[ks], dh[C0 + c]);
        }
      }
      f16x8 fp[G::NB][KB];
      f16x4 fl[G::NB][G::NB], ft[G::NB];
      f32x4 bz[G::NB];
#pragma unroll
      for (int J = 0; J < G::NB; ++J) {
#pragma unroll
        for (int ks = 0; ks < KB; ++ks)
          if (32 * ks + 31 >= 16 * J) fp[J][ks] = lds_a_perm_tr_sw<BC>(&s.P[0][0], 32 * ks, 16 * J, HALF);
        ft[J] = lds_tr4(&s.Td[0][0], 24, 16 * J, 0);
#pragma unroll
        for (int I = 0; I < J; ++I) fl[I][J] = lds_tr4_sw<BC>(&s.L[0][0], 16 * J, 16 * I);  // block (I, J) of -A^T
#pragma unroll
        for (int r = 0; r < 4; ++r) bz[J][r] = s.beta[16 * J + 4 * g + r];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int J = 0; J < G::NB; ++J)
#pragma unroll
        for (int ks = 0; ks < KB; ++ks)
          if (32 * ks + 31 >= 16 * J) dd[J] = mfma16(fp[J][ks], dob[ks], dd[J]);
      // (I + diag(beta) A)^T dy = ddelta, from the last block up:
      // dy_I = Td_I^T (ddelta_I - sum_{J>I} A_JI^T diag(beta_J) dy_J)
      f32x4 w[G::NB];
#pragma unroll
      for (int I = G::NB - 1; I >= 0; --I) {
        f32x4 rr = dd[I];
#pragma unroll
        for (int J = G::NB - 1; J > I; --J) rr = mfma16k16(fl[I][J], acc4(w[J]), rr);
        f32x4 dy = mfma16k16(ft[I], acc4(rr), (f32x4){0.f, 0.f, 0.f, 0.f});
        w[I] = dy * bz[I];
        // rows past the chunk are masked by the reader
        if (16 * I < len) st_h4(a.dy + blk * (BC * D) + state_tile<D>(I, col >> 4), dy);
      }
      f16x8 wb[KB];
#pragma unroll
      for (int ks = 0; ks < KB; ++ks) wb[ks] = HALF ? acc_half(w[0]) : acc_pair(w[2 * ks], w[2 * ks + 1]);
      // dh -= (K e^Gam)^T diag(beta) dy
#pragma unroll
      for (int C0 = 0; C0 < G::NCB; C0 += HC) {
        f16x8 fb[HC][KB];
#pragma unroll
        for (int c = 0; c < HC; ++c)
#pragma unroll
          for (int ks = 0; ks < KB; ++ks) fb[c][ks] = lds_a_perm_tr_sw<D>(&s.Kn[0][0], 32 * ks, 16 * (C0 + c), HALF);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < HC; ++c)
#pragma unroll
          for (int ks = 0; ks < KB; ++ks) dh[C0 + c] = mfma16(fb[c][ks], wb[ks], dh[C0 + c]);
      }
    }
  }
  if (sw) {   // the start-state gradient, unscaled, and its largest magnitude
    float* dst = a.slot + ((size_t)seq * H + h) * DD;
    float mx = 0.f;
#pragma unroll
    for (int C = 0; C < G::NCB; ++C)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = inv * dh[C][r];
        dst[(size_t)(16 * C + 4 * g + r) * D + col] = x;
        mx = fmaxf(mx, fabsf(x));
      }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if (lane == 0 && mx > 0.f)
      atomicMax(slot_words(a.gmax, a.n_rounds, round) + (blockIdx.x * NW + wave) % SPREAD,
                __float_as_uint(mx));
  }
}

// dO of every chunk-head in 16x16 tiles (state_tile order, chunk.h): row i
// of chunk c holds dO[out_row[chunk_row0[c] + i]] for rows with an output,
// zero on replay rows and past the chunk.  One block per chunk-head: its rows
// are read whole into LDS (16-byte pieces, a wave per 4 or 2 rows), then the
// tiles are written in their own order (a wave per contiguous tile).
template <typename TIn, int BC, int D>
__global__ __launch_bounds__(256) void k_gather_dO(const TIn* dO, DevPlan plan, int H, TIn* dOp,
                                                   int c_begin, unsigned* gmax) {
  constexpr int PER = 16 / (int)sizeof(TIn);  // elements per 16-byte piece: 8 or 4
  constexpr int PPR = D / PER;                // pieces per row
  constexpr int PITCH = D + PER;              // LDS row pitch, padded by one piece
  using V = TIn __attribute__((ext_vector_type(PER)));
  using V4 = in4_t<TIn>;
  __shared__ __attribute__((aligned(16))) TIn rowsm[BC * PITCH];
  __shared__ float wmax[4];
  const int c = c_begin + blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int row0 = ld_uni(plan.chunk_row0, c), len = ld_uni(plan.chunk_len, c);
  float mx = 0.f;   // largest |dO| of the chunk-head, for its round's gradient scale
  for (int p = tid; p < BC * PPR; p += 256) {
    const int i = p / PPR, j = p % PPR;
    const int o = i < len ? plan.out_row[row0 + i] : -1;
    V x = (V)0;
    if (o >= 0) x = *(const V*)&dO[((size_t)o * H + h) * D + j * PER];
    *(V*)&rowsm[i * PITCH + j * PER] = x;
#pragma unroll
    for (int e = 0; e < PER; ++e) mx = fmaxf(mx, fabsf(in_f32(x[e])));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((tid & 63) == 0) wmax[tid >> 6] = mx;
  __syncthreads();
  if (tid == 0) {
    mx = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    if (mx > 0.f)
      atomicMax(dO_words(gmax, ld_uni(plan.chunk_round, c)) + (blockIdx.x + 7 * blockIdx.y) % SPREAD,
                __float_as_uint(mx));
  }
  TIn* dst = dOp + ((size_t)c * H + h) * (BC * D);
  for (int q = tid; q < BC * D / 4; q += 256) {   // lane l of tile t: its accumulator piece
    const int t = q >> 6, l = q & 63;
    const int i = 16 * (t / (D / 16)) + 4 * (l >> 4);
    const int v = 16 * (t % (D / 16)) + (l & 15);
    V4 x;
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = rowsm[(i + r) * PITCH + v];
    *(V4*)&dst[4 * (size_t)q] = x;
  }
}

// chunks c_begin .. c_begin + n_chunks - 1
hipError_t launch_gather_dO(const BwdArgs& a, bool bf16, int BC, int D, int c_begin, int n_chunks,
                            hipStream_t st) {
  if (n_chunks <= 0) return hipSuccess;
#define KDA_GDO(T, BCv, Dv)                                                                    \
  if (BC == BCv && D == Dv) {                                                                  \
    KDA_LAUNCH("kda_bwd_gather_dO", (k_gather_dO<T, BCv, Dv>), dim3(n_chunks, a.H), dim3(256), \
               st, (const T*)a.dO, a.plan, a.H, (T*)a.dOp, c_begin, a.gmax);                   \
    return hipGetLastError();                                                                  \
  }
  if (bf16) {
    KDA_GDO(uint16_t, 64, 128) KDA_GDO(uint16_t, 64, 64) KDA_GDO(uint16_t, 16, 128)
    KDA_GDO(uint16_t, 16, 64)
  } else {
    KDA_GDO(float, 64, 128) KDA_GDO(float, 64, 64) KDA_GDO(float, 16, 128) KDA_GDO(float, 16, 64)
  }
#undef KDA_GDO
  return hipErrorInvalidValue;
}

int round_slices(int nseq, int H, int D, int max_slices);

template <typename TIn, int BC, int D, int NV>
hipError_t launch_bround(const BwdArgs& a, int nseq, int seq0, int round, int slices,
                         hipStream_t st) {
  KDA_LAUNCH("kda_bwd_round", (k_bwd_round<TIn, BC, D, NV>), dim3(nseq * a.H, 1, slices), dim3(NT),
             st, a, seq0, round);
  return hipGetLastError();
}

template <typename TIn, int BC, int D>
hipError_t launch_brounds_t(const BwdArgs& a, const int* round_ptr_host, int r_begin, int r_end,
                            int max_slices, hipStream_t st) {
  constexpr int NCB = D / 16;
  for (int r = r_end - 1; r >= r_begin; --r) {
    const int nseq = round_ptr_host[r + 1] - round_ptr_host[r];
    if (nseq == 0) continue;
    const int sl = round_slices(nseq, a.H, D, max_slices);
    const int nv = NCB / sl;
    hipError_t e = hipErrorInvalidValue;
    if (nv == NCB) e = launch_bround<TIn, BC, D, NCB>(a, nseq, round_ptr_host[r], r, sl, st);
    else if (nv == 4) e = launch_bround<TIn, BC, D, 4>(a, nseq, round_ptr_host[r], r, sl, st);
    else if (nv == 2) e = launch_bround<TIn, BC, D, 2>(a, nseq, round_ptr_host[r], r, sl, st);
    else if (nv == 1) e = launch_bround<TIn, BC, D, 1>(a, nseq, round_ptr_host[r], r, sl, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// rounds r_end - 1 down to r_begin
hipError_t launch_bwd_rounds(const BwdArgs& a, bool bf16, int BC, int D, const int* round_ptr_host,
                             int r_begin, int r_end, int max_slices, hipStream_t st) {
#define KDA_BR_CASE(T, BCv, Dv) \
  if (BC == BCv && D == Dv) \
    return launch_brounds_t<T, BCv, Dv>(a, round_ptr_host, r_begin, r_end, max_slices, st);
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
