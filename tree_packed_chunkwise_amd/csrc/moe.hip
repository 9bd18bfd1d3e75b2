// moe.hip -- occurrence-weighted router statistics over compact rows (gfx950).
//
// HARTS abstract: for deterministic top-k routing without token dropping,
// occurrence counts restore MoE objective weights and expert-load
// statistics; thelatestinai.com Figure 1 caption (occurrence count q_B = 2
// of a row shared by two trajectories) and Figure C.1(d) (compact routing
// with multiplicity-weighted router losses and expert-load counts).  A
// compact row read by q trajectory positions contributes q times what one
// position contributes to the statistics of the trajectory-expanded batch:
//   load[e] = sum_r q_r [e in topk(x_r)]          (exact integers)
//   psum[e] = sum_r q_r softmax(x_r)[e]
//   zsum    = sum_r q_r logsumexp(x_r)^2,   n_tok = sum_r q_r
// and, in reverse, dx_r = q_r (p_r (g - <p_r, g>) + 2 gz lse_r p_r).
// Top-k: the k largest logits, equal logits ordered by the lower expert index.
//
//   k_router_stats  one wave per row (E / 64 experts per lane): softmax and
//                   logsumexp by wave reductions, top-k by a radix select on
//                   order-preserving keys (ballots and scalar popcounts);
//                   per-block sums over a fixed range of rows, waves combined
//                   in a fixed order
//   k_router_sum    block partials summed per column in a fixed order
//                   (strided per thread, then an LDS tree: deterministic)
//   k_router_bwd    one wave per row: the reverse-mode row above
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "timing.h"

namespace kda {

constexpr int MT = 256;        // threads per block (4 waves)
constexpr int MW = MT / 64;

__device__ inline float ld_x(const float* p, size_t i) { return p[i]; }
__device__ inline float ld_x(const uint16_t* p, size_t i) {
  return __uint_as_float(((uint32_t)p[i]) << 16);
}

// Wave-wide reductions without an LDS round trip: DPP quad permutes and row
// mirrors inside each 16-lane row, then gfx950's row swaps across rows.  Each
// step pairs every lane with one partner (an involution), so a symmetric
// combine leaves the same result in every lane.
template <int CTRL>
__device__ inline float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <typename F>
__device__ inline float wave_reduce(float v, F op) {
  v = op(v, dpp_f<0xB1>(v));    // quad_perm [1,0,3,2]
  v = op(v, dpp_f<0x4E>(v));    // quad_perm [2,3,0,1]
  v = op(v, dpp_f<0x141>(v));   // row_half_mirror
  v = op(v, dpp_f<0x140>(v));   // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float wave_max(float v) {
  return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}
__device__ inline float wave_sum(float v) {
  return wave_reduce(v, [](float a, float b) { return a + b; });
}

// Order-preserving key of a logit (larger value, larger key; -0 keys as +0,
// which compares equal to it), kept to the bits the input type can vary:
// the high 16 of a bf16 value.
template <typename T> struct KeyBits { static constexpr int n = 32; };
template <> struct KeyBits<uint16_t> { static constexpr int n = 16; };
template <typename T>
__device__ inline uint32_t order_key(float f) {
  const uint32_t u = f == 0.f ? 0u : __float_as_uint(f);
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return k >> (32 - KeyBits<T>::n);
}

// rows per block: a fixed function of the row count (so the partial sums,
// and with them the results, do not depend on the launch)
inline int64_t router_rows_per_block(int64_t n_rows) {
  const int64_t r = (n_rows + 2047) / 2048;
  return r < 64 ? 64 : r;
}
inline int64_t router_blocks(int64_t n_rows) {
  const int64_t rpb = router_rows_per_block(n_rows);
  return (n_rows + rpb - 1) / rpb;
}

// ws: float part[nblk][E + 1] (psum, zsum) | int part[nblk][E + 1] (load, n_tok)
template <typename T_, int EPL>
__global__ __launch_bounds__(MT) void k_router_stats(const T_* x, const int* q, int64_t n_rows,
                                                     int k, int64_t rpb, int* tidx, float* tprob,
                                                     float* partf, int* parti) {
  constexpr int E = 64 * EPL;
  __shared__ float sf[MW][E + 1];
  __shared__ int si[MW][E + 1];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t r0 = (int64_t)blockIdx.x * rpb;
  const int64_t r1 = r0 + rpb < n_rows ? r0 + rpb : n_rows;
  float accp[EPL], accz = 0.f;
  int accc[EPL], acct = 0;
#pragma unroll
  for (int j = 0; j < EPL; ++j) { accp[j] = 0.f; accc[j] = 0; }
  for (int64_t row = r0 + wave; row < r1; row += MW) {
    const int qr = q[row];
    float v[EPL], p[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) v[j] = ld_x(x, (size_t)row * E + lane + 64 * j);
    float m = v[0];
#pragma unroll
    for (int j = 1; j < EPL; ++j) m = fmaxf(m, v[j]);
    m = wave_max(m);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) s += __expf(v[j] - m);
    const float lse = m + __logf(wave_sum(s));
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      p[j] = __expf(v[j] - lse);
      accp[j] += (float)qr * p[j];
    }
    accz += (float)qr * lse * lse;
    acct += qr;
    // top-k by radix select on order-preserving keys: the k-th largest key
    // T bit by bit (one ballot and popcount per bit), every key above T, and
    // the ties at T of the lowest experts
    uint32_t key[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) key[j] = order_key<T_>(v[j]);
    uint32_t T = 0u;
    for (int b = KeyBits<T_>::n - 1; b >= 0; --b) {
      const uint32_t c = T | (1u << b);
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < EPL; ++j) cnt += __popcll(__ballot(key[j] >= c));
      if (cnt >= k) T = c;
    }
    int gt = 0;
#pragma unroll
    for (int j = 0; j < EPL; ++j) gt += __popcll(__ballot(key[j] > T));
    bool sel[EPL];
    unsigned long long selm[EPL];
    {
      int ties_before = 0;   // ties at T held by lower experts (lower j, then lower lane)
      const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const unsigned long long eq = __ballot(key[j] == T);
        const int rank_eq = ties_before + __popcll(eq & below);
        sel[j] = key[j] > T || (key[j] == T && rank_eq < k - gt);
        ties_before += __popcll(eq);
        selm[j] = __ballot(sel[j]);
        if (sel[j]) accc[j] += qr;
      }
    }
    if (tidx || tprob) {
      // output order: rank = chosen experts before this one (larger key, or
      // the same key and a lower expert), by broadcasting the k chosen
      int rank[EPL];
#pragma unroll
      for (int j = 0; j < EPL; ++j) rank[j] = 0;
#pragma unroll
      for (int js = 0; js < EPL; ++js) {
        unsigned long long m = selm[js];
        while (m) {
          const int ls = __builtin_ctzll(m);
          m &= m - 1ull;
          const uint32_t ks = (uint32_t)__builtin_amdgcn_readlane((int)key[js], ls);
          const int es = ls + 64 * js;
#pragma unroll
          for (int j = 0; j < EPL; ++j)
            rank[j] += (ks > key[j] || (ks == key[j] && es < lane + 64 * j)) ? 1 : 0;
        }
      }
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (sel[j]) {
          if (tidx) tidx[row * k + rank[j]] = lane + 64 * j;
          if (tprob) tprob[row * k + rank[j]] = p[j];
        }
    }
  }
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    sf[wave][lane + 64 * j] = accp[j];
    si[wave][lane + 64 * j] = accc[j];
  }
  if (lane == 0) {
    sf[wave][E] = accz;
    si[wave][E] = acct;
  }
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += MT) {
    float a = 0.f;
    int b = 0;
#pragma unroll
    for (int w = 0; w < MW; ++w) {
      a += sf[w][e];
      b += si[w][e];
    }
    partf[(size_t)blockIdx.x * (E + 1) + e] = a;
    parti[(size_t)blockIdx.x * (E + 1) + e] = b;
  }
}

// one block per column (expert, then the z-loss / count column): thread t
// sums the partials t, t + MT, ... in order, then a fixed LDS tree
__global__ __launch_bounds__(MT) void k_router_sum(const float* partf, const int* parti, int nblk,
                                                   int E, float* psum, int64_t* load, float* zsum,
                                                   int64_t* n_tok) {
  __shared__ float sa[MT];
  __shared__ int64_t sb[MT];
  const int e = blockIdx.x, t = threadIdx.x;
  float a = 0.f;
  int64_t b = 0;
  for (int i = t; i < nblk; i += MT) {
    a += partf[(size_t)i * (E + 1) + e];
    b += parti[(size_t)i * (E + 1) + e];
  }
  sa[t] = a;
  sb[t] = b;
  __syncthreads();
  for (int h = MT / 2; h > 0; h >>= 1) {
    if (t < h) {
      sa[t] += sa[t + h];
      sb[t] += sb[t + h];
    }
    __syncthreads();
  }
  if (t == 0) {
    if (e < E) {
      psum[e] = sa[0];
      load[e] = sb[0];
    } else {
      *zsum = sa[0];
      *n_tok = sb[0];
    }
  }
}

template <typename T, int EPL>
__global__ __launch_bounds__(MT) void k_router_bwd(const T* x, const int* q, int64_t n_rows,
                                                   const float* g, float gz, float* dx) {
  constexpr int E = 64 * EPL;
  const int lane = threadIdx.x & 63;
  float gl[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) gl[j] = g[lane + 64 * j];
  const int64_t nw = (int64_t)gridDim.x * MW;
  for (int64_t row = (int64_t)blockIdx.x * MW + (threadIdx.x >> 6); row < n_rows; row += nw) {
    const float qr = (float)q[row];
    float v[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) v[j] = ld_x(x, (size_t)row * E + lane + 64 * j);
    float m = v[0];
#pragma unroll
    for (int j = 1; j < EPL; ++j) m = fmaxf(m, v[j]);
    m = wave_max(m);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) s += __expf(v[j] - m);
    const float lse = m + __logf(wave_sum(s));
    float p[EPL], d = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      p[j] = __expf(v[j] - lse);
      d += p[j] * gl[j];
    }
    d = wave_sum(d);
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      dx[(size_t)row * E + lane + 64 * j] = qr * p[j] * (gl[j] - d + 2.f * gz * lse);
  }
}

size_t router_ws_bytes(int64_t n_rows, int E) {
  return (size_t)router_blocks(n_rows) * (E + 1) * 8;
}

// Scratch of moe_router_stats_noalloc: the block partials of the largest
// launch (2048 blocks, 512 experts), in a device array of the library, so
// that the call allocates nothing.  Each device holds its own copy for the
// life of the process; its address is looked up once per device (the name
// itself is only a host-side handle).  Calls on one device share it.
constexpr size_t kRouterScratchBytes = (size_t)2048 * (512 + 1) * 8;
static __device__ __align__(256) unsigned char scratch[kRouterScratchBytes];

hipError_t router_scratch(void** ptr, size_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {   // first call on this device, with it current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = kRouterScratchBytes;
  return hipSuccess;
}

hipError_t launch_router_stats(const void* x, bool bf16, int64_t n_rows, int E, int k,
                               const int* q, int* tidx, float* tprob, int64_t* load, float* psum,
                               float* zsum, int64_t* n_tok, void* ws, hipStream_t st) {
  const int64_t rpb = router_rows_per_block(n_rows);
  const int nblk = (int)router_blocks(n_rows);
  float* partf = (float*)ws;
  int* parti = (int*)(partf + (size_t)nblk * (E + 1));
  if (nblk > 0) {
#define KDA_RS(T, EPLv)                                                                          \
  KDA_LAUNCH("moe_router_stats", (k_router_stats<T, EPLv>), dim3(nblk), dim3(MT), st,             \
             (const T*)x, q, n_rows, k, rpb, tidx, tprob, partf, parti)
    const int epl = E / 64;
    if (bf16) {
      if (epl == 1) KDA_RS(uint16_t, 1); else if (epl == 2) KDA_RS(uint16_t, 2);
      else if (epl == 4) KDA_RS(uint16_t, 4); else KDA_RS(uint16_t, 8);
    } else {
      if (epl == 1) KDA_RS(float, 1); else if (epl == 2) KDA_RS(float, 2);
      else if (epl == 4) KDA_RS(float, 4); else KDA_RS(float, 8);
    }
#undef KDA_RS
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  KDA_LAUNCH("moe_router_sum", k_router_sum, dim3(E + 1), dim3(MT), st, partf, parti, nblk, E, psum,
             load, zsum, n_tok);
  return hipGetLastError();
}

hipError_t launch_router_bwd(const void* x, bool bf16, int64_t n_rows, int E, const int* q,
                             const float* g, float gz, float* dx, hipStream_t st) {
  if (n_rows <= 0) return hipSuccess;
  const int64_t want = (n_rows + MW - 1) / MW;
  const int nb = (int)(want < 65536 ? want : 65536);
#define KDA_RB(T, EPLv)                                                                            \
  KDA_LAUNCH("moe_router_bwd", (k_router_bwd<T, EPLv>), dim3(nb), dim3(MT), st, (const T*)x, q,     \
             n_rows, g, gz, dx)
  const int epl = E / 64;
  if (bf16) {
    if (epl == 1) KDA_RB(uint16_t, 1); else if (epl == 2) KDA_RB(uint16_t, 2);
    else if (epl == 4) KDA_RB(uint16_t, 4); else KDA_RB(uint16_t, 8);
  } else {
    if (epl == 1) KDA_RB(float, 1); else if (epl == 2) KDA_RB(float, 2);
    else if (epl == 4) KDA_RB(float, 4); else KDA_RB(float, 8);
  }
#undef KDA_RB
  return hipGetLastError();
}

}  // namespace kda
