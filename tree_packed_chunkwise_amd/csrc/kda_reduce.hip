// kda_reduce.hip -- the two fixed-order reductions that close the reverse
// pass (gfx950), after the state-gradient rounds and the chunk-local
// gradients of every chunk (launch order in schedule.cpp):
//   - gradients of replayed rows (rows a side sequence recomputes from the
//     start of its chunk, HARTS Figure 2(c)) added into their compact rows;
//   - dh0 of every root: the sum of the start-state gradients of the
//     sequences that start from it.
// Both reductions add in a fixed order, so results do not depend on timing.
// Also the pass before the rounds that clears the reverse call's
// gradient-scale words and finds the largest leaf-state gradient (common.h).
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
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int p = p0; p < p1; ++p) {
    const float4 x = ((const float4*)(a.slot + ((size_t)a.plan.root_seq[p] * H + h) * (4 * DD4)))[e4];
    acc.x += x.x;
    acc.y += x.y;
    acc.z += x.z;
    acc.w += x.w;
  }
  ((float4*)(a.dh0 + ((size_t)rt * H + h) * (4 * DD4)))[e4] = acc;
}

// The gradient-scale words of a reverse call (common.h): cleared, then the
// largest |dh_leaf| (16-byte loads, four in flight per thread, a block
// maximum, one integer atomic max per block on a spread word).
__global__ __launch_bounds__(BT) void k_zero_words(unsigned* w, int n) {
  for (int i = threadIdx.x; i < n; i += BT) w[i] = 0u;
}

__global__ __launch_bounds__(BT) void k_leaf_absmax(const float* dhl, size_t n, unsigned* gmax) {
  constexpr int U = 4;
  __shared__ float red[BT / 64];
  const size_t stride = (size_t)gridDim.x * BT * U;
  const size_t t0 = (size_t)blockIdx.x * BT * U + threadIdx.x;
  const float4* s4 = (const float4*)dhl;
  const size_t n4 = n / 4;
  float m = 0.f;
  for (size_t i = t0; i < n4; i += stride) {
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = i + (size_t)u * BT < n4 ? s4[i + (size_t)u * BT] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < U; ++u)
      m = fmaxf(m, fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w))));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < BT / 64; ++w) m = fmaxf(m, red[w]);
    if (m > 0.f) atomicMax(leaf_words(gmax) + blockIdx.x % SPREAD, __float_as_uint(m));
  }
}

// n_dhl elements of dh_leaf (a multiple of 4; dh_leaf may be null)
hipError_t launch_scale_words(const BwdArgs& a, size_t n_dhl, hipStream_t st) {
  KDA_LAUNCH("kda_bwd_grad_scale", k_zero_words, dim3(1), dim3(BT), st, a.gmax,
             (int)scale_words(a.n_rounds));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.dh_leaf || n_dhl == 0) return e;
  size_t nb = (n_dhl / 16 + BT - 1) / BT;
  nb = nb < 1 ? 1 : (nb > 2048 ? 2048 : nb);
  KDA_LAUNCH("kda_bwd_grad_scale", k_leaf_absmax, dim3((unsigned)nb), dim3(BT), st, a.dh_leaf,
             n_dhl, a.gmax);
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
