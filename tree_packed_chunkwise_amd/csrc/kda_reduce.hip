// kda_reduce.hip -- the two fixed-order reductions that close the reverse
// pass (gfx950), after the state-gradient rounds and the chunk-local
// gradients of every chunk (launch order in schedule.cpp):
//   - gradients of replayed rows (rows a side sequence recomputes from the
//     start of its chunk, HARTS Figure 2(c)) added into their compact rows;
//   - dh0 of every root: the sum of the start-state gradients of the
//     sequences that start from it.
// Both reductions add in a fixed order, so results do not depend on timing.
// Also the pass before the rounds that finds the reverse call's power-of-two
// scale (the largest upstream gradient, bwd_scale in common.h).
#include "common.h"
#include "timing.h"

namespace kda {

constexpr int BT = 256;  // threads per block of the dh0 reduction

// replayed-row gradients added into their compact rows (fixed order); one
// thread per channel
template <int D>
__global__ __launch_bounds__(D) void k_reduce_rep(BwdArgs a) {
  const int e = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int H = a.H;
  const int row = a.plan.rep_row[e];
  const int p0 = a.plan.rep_ptr[e], p1 = a.plan.rep_ptr[e + 1];
  {
    const int ch = tid;
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

// dh0 of every root: sum of the start gradients of its sequences (fixed
// order); one float4 of one (root, head) state per thread
template <int D>
__global__ __launch_bounds__(BT) void k_reduce_dh0(BwdArgs a) {
  constexpr int DD4 = D * D / 4;
  const int rh = blockIdx.y, H = a.H, rt = rh / H, h = rh % H;
  const int e4 = blockIdx.x * BT + threadIdx.x;   // grid.x * BT == DD4
  const int p0 = a.plan.root_seq_ptr[rt], p1 = a.plan.root_seq_ptr[rt + 1];
  const float inv = 1.f / bwd_scale(a.gmax, a.scale);   // the slots are in scaled units
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int p = p0; p < p1; ++p) {
    const float4 x = ((const float4*)(a.slot + ((size_t)a.plan.root_seq[p] * H + h) * (4 * DD4)))[e4];
    acc.x += x.x;
    acc.y += x.y;
    acc.z += x.z;
    acc.w += x.w;
  }
  ((float4*)(a.dh0 + ((size_t)rt * H + h) * (4 * DD4)))[e4] =
      make_float4(inv * acc.x, inv * acc.y, inv * acc.z, inv * acc.w);
}

// The largest |dO| and |dh_leaf| of a reverse call (bwd_scale, common.h):
// 16-byte loads, a wave maximum, one integer atomic max per wave on the fp32
// bits (non-negative floats order like their bits, and a maximum does not
// depend on the order of the updates, so the result is deterministic).
__global__ __launch_bounds__(64) void k_zero_gmax(unsigned* gmax) {
  if (threadIdx.x < 2) gmax[threadIdx.x] = 0u;
}

__device__ inline float elem_f32(float x) { return x; }
__device__ inline float elem_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

template <typename TIn>
__global__ __launch_bounds__(BT) void k_absmax(const TIn* dO, size_t n_do, const float* dhl,
                                               size_t n_dhl, unsigned* gmax) {
  typedef __attribute__((__vector_size__(16))) unsigned u4;
  constexpr int PER = 16 / (int)sizeof(TIn);
  const size_t stride = (size_t)gridDim.x * BT, t0 = (size_t)blockIdx.x * BT + threadIdx.x;
  float m0 = 0.f, m1 = 0.f;
  for (size_t i = t0; i < n_do / PER; i += stride) {
    const u4 v = ((const u4*)dO)[i];
    const TIn* e = (const TIn*)&v;
#pragma unroll
    for (int j = 0; j < PER; ++j) m0 = fmaxf(m0, fabsf(elem_f32(e[j])));
  }
  if (dhl) {
    for (size_t i = t0; i < n_dhl / 4; i += stride) {
      const float4 v = ((const float4*)dhl)[i];
      m1 = fmaxf(m1, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    m0 = fmaxf(m0, __shfl_xor(m0, o));
    m1 = fmaxf(m1, __shfl_xor(m1, o));
  }
  if ((threadIdx.x & 63) == 0) {
    atomicMax(&gmax[0], __float_as_uint(m0));
    atomicMax(&gmax[1], __float_as_uint(m1));
  }
}

// n_do elements of dO (a multiple of 16 / sizeof(element)), n_dhl of dh_leaf
// (a multiple of 4; dh_leaf may be null)
hipError_t launch_absmax(const BwdArgs& a, bool bf16, size_t n_do, size_t n_dhl, hipStream_t st) {
  KDA_LAUNCH("kda_bwd_grad_scale", k_zero_gmax, dim3(1), dim3(64), st, a.gmax);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t n = n_do > n_dhl ? n_do : n_dhl;
  size_t nb = (n / 8 + BT - 1) / BT;
  nb = nb < 1 ? 1 : (nb > 2048 ? 2048 : nb);
  if (bf16)
    KDA_LAUNCH("kda_bwd_grad_scale", k_absmax<uint16_t>, dim3((unsigned)nb), dim3(BT), st,
               (const uint16_t*)a.dO, n_do, a.dh_leaf, n_dhl, a.gmax);
  else
    KDA_LAUNCH("kda_bwd_grad_scale", k_absmax<float>, dim3((unsigned)nb), dim3(BT), st,
               (const float*)a.dO, n_do, a.dh_leaf, n_dhl, a.gmax);
  return hipGetLastError();
}

template <int D>
hipError_t launch_reduce_t(const BwdArgs& a, int n_rep_rows, int n_root, hipStream_t st) {
  if (n_rep_rows > 0) {
    KDA_LAUNCH("kda_bwd_reduce_replay", (k_reduce_rep<D>), dim3(n_rep_rows, a.H), dim3(D), st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (n_root > 0) {
    static_assert((D * D / 4) % BT == 0, "whole blocks");
    KDA_LAUNCH("kda_bwd_reduce_dh0", (k_reduce_dh0<D>), dim3(D * D / 4 / BT, n_root * a.H), dim3(BT),
               st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_reduce(const BwdArgs& a, int D, int n_rep_rows, int n_root, hipStream_t st) {
  if (D != 64 && D != 128) return hipErrorInvalidValue;
  return D == 128 ? launch_reduce_t<128>(a, n_rep_rows, n_root, st)
                  : launch_reduce_t<64>(a, n_rep_rows, n_root, st);
}

}  // namespace kda
