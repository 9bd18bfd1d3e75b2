// gather.hip -- per-original-position log-probs from compact logit rows (gfx950).
//
// HARTS abstract: log-probabilities are recovered for each original
// trajectory position; Figure 1: one logit row serves several trajectories'
// distinct targets; Figure C.1(d): no expanded vocabulary-sized logits.
//
//   k_row_lse   one block per compact row: online max / sum-of-exp over the
//               vocabulary in one pass (16-byte loads, one rescale per load),
//               fixed-order tree reduction -> lse[row]
//   k_pos_logp  one thread per position: logits[row, tgt] - lse[row]
//   k_row_grad  one block per compact row: w = sum of the row's dlogp (CSR
//               order); every element -softmax * w (16-byte loads and
//               stores), then the row's target
//               columns get their exact value (-softmax*w + sum of dlogp of the
//               positions targeting that column), one position per thread.
// HBM-bound: each logit is read once per pass and each gradient written once.
//
// Masked entries: a logit of -inf has probability zero (it adds nothing to
// the row's sum of exponentials and its softmax value is 0).  A row whose
// every entry is -inf has lse = -inf, every position on it gets logp = -inf,
// and its softmax is taken as all zeros (only the target columns of its
// gradient are nonzero).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "timing.h"

namespace kda {

constexpr int GT = 256;

__device__ inline float ld_logit(const float* p, size_t i) { return p[i]; }
__device__ inline float ld_logit(const uint16_t* p, size_t i) {
  return __uint_as_float(((uint32_t)p[i]) << 16);
}
__device__ inline void st_logit(float* p, size_t i, float x) { p[i] = x; }
__device__ inline void st_logit(uint16_t* p, size_t i, float x) {
  p[i] = __builtin_bit_cast(uint16_t, (__bf16)x);
}

// running (max, sum of exp(x - max)); (-inf, 0) until a finite logit arrives,
// and -inf logits add nothing (exp(-inf - m) would be NaN while m = -inf)
__device__ inline void online_add(float& m, float& s, float x) {
  if (x > m) {
    s = s * __expf(m - x) + 1.f;
    m = x;
  } else if (x > -INFINITY) {
    s += __expf(x - m);
  }
}

__device__ inline void online_merge(float& m, float& s, float m2, float s2) {
  if (m2 > m) {
    s = s * __expf(m - m2) + s2;
    m = m2;
  } else if (m2 > -INFINITY) {
    s += s2 * __expf(m2 - m);
  }
}

// a run of n logits into (m, s) at once: one rescale for the run's maximum,
// then its exponentials (-inf logits add nothing; an all -inf run changes nothing)
template <int N>
__device__ inline void online_add_run(float& m, float& s, const float (&x)[N]) {
  float mx = x[0];
#pragma unroll
  for (int j = 1; j < N; ++j) mx = __builtin_fmaxf(mx, x[j]);
  if (mx == -INFINITY) return;
  if (mx > m) {
    s *= __expf(m - mx);   // 0 while m = -inf
    m = mx;
  }
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < N; ++j) t += __expf(x[j] - m);
  s += t;
}

template <typename T>
__device__ inline void row_stats(const T* z, int vocab, float& m, float& s, float* sm, float* ss) {
  m = -INFINITY;
  s = 0.f;
  const int tid = threadIdx.x;
  constexpr int VEC = 16 / sizeof(T);
  const int nvec = vocab / VEC;
  if ((((uintptr_t)z) % 16) == 0) {
    typedef __attribute__((__vector_size__(16))) int v4i;
    const v4i* zv = (const v4i*)z;
#pragma unroll 2
    for (int i = tid; i < nvec; i += GT) {
      v4i pk = zv[i];
      const T* e = (const T*)&pk;
      float x[VEC];
#pragma unroll
      for (int j = 0; j < VEC; ++j) x[j] = ld_logit(e, j);
      online_add_run(m, s, x);
    }
    for (int i = nvec * VEC + tid; i < vocab; i += GT) online_add(m, s, ld_logit(z, i));
  } else {
    for (int i = tid; i < vocab; i += GT) online_add(m, s, ld_logit(z, i));
  }
  sm[tid] = m;
  ss[tid] = s;
  __syncthreads();
  for (int w = GT / 2; w > 0; w >>= 1) {
    if (tid < w) {
      float a = sm[tid], b = ss[tid];
      online_merge(a, b, sm[tid + w], ss[tid + w]);
      sm[tid] = a;
      ss[tid] = b;
    }
    __syncthreads();
  }
  m = sm[0];
  s = ss[0];
}

template <typename T>
__global__ __launch_bounds__(GT) void k_row_lse(const T* logits, int vocab, float* lse) {
  __shared__ float sm[GT], ss[GT];
  const size_t row = blockIdx.x;
  float m, s;
  row_stats(logits + row * vocab, vocab, m, s, sm, ss);
  if (threadIdx.x == 0) lse[row] = m + __logf(s);
}

template <typename T>
__global__ void k_pos_logp(const T* logits, int vocab, const int* pos_row, const int* pos_tgt,
                           int64_t n_pos, const float* lse, float* logp) {
  const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= n_pos) return;
  const int r = pos_row[p];
  const float l = lse[r];
  logp[p] = l == -INFINITY ? -INFINITY : ld_logit(logits, (size_t)r * vocab + pos_tgt[p]) - l;
}

template <typename T>
__global__ __launch_bounds__(GT) void k_row_grad(const T* logits, int vocab, const float* lse,
                                                 const int* row_pos_ptr, const int* row_pos_idx,
                                                 const int* pos_tgt, const float* dlogp,
                                                 T* dlogits) {
  const size_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int p0 = row_pos_ptr[row], p1 = row_pos_ptr[row + 1];
  float w = 0.f;
  for (int p = p0; p < p1; ++p) w += dlogp[row_pos_idx[p]];
  const float l = lse[row];
  const bool dead = l == -INFINITY;   // every entry masked: softmax taken as 0
  const T* z = logits + row * vocab;
  T* dz = dlogits + row * vocab;
  int done = 0;   // elements the 16-byte loop covers
  if (((((uintptr_t)z) | ((uintptr_t)dz)) % 16) == 0) {
    typedef __attribute__((__vector_size__(16))) int v4i;
    constexpr int VEC = 16 / sizeof(T);
    const int nvec = vocab / VEC;
#pragma unroll 2
    for (int i = tid; i < nvec; i += GT) {
      const v4i pk = ((const v4i*)z)[i];
      v4i out;
      const T* e = (const T*)&pk;
      T* o = (T*)&out;
#pragma unroll
      for (int j = 0; j < VEC; ++j) st_logit(o, j, dead ? 0.f : -__expf(ld_logit(e, j) - l) * w);
      ((v4i*)dz)[i] = out;
    }
    done = nvec * VEC;
  }
  for (int i = done + tid; i < vocab; i += GT)
    st_logit(dz, i, dead ? 0.f : -__expf(ld_logit(z, i) - l) * w);
  __syncthreads();
  // target columns, one position per thread: positions sharing a target sum
  // the same terms in the same (CSR) order and write the same value
  for (int q = p0 + tid; q < p1; q += GT) {
    const int t = pos_tgt[row_pos_idx[q]];
    float acc = dead ? 0.f : -__expf(ld_logit(z, t) - l) * w;
    for (int p2 = p0; p2 < p1; ++p2)
      if (pos_tgt[row_pos_idx[p2]] == t) acc += dlogp[row_pos_idx[p2]];
    st_logit(dz, t, acc);
  }
}

hipError_t launch_gather_fwd(const void* logits, bool bf16, int64_t n_rows, int vocab,
                             const int* pos_row, const int* pos_tgt, int64_t n_pos, float* logp,
                             float* lse, hipStream_t st) {
  if (n_rows > 0) {
    if (bf16)
      KDA_LAUNCH("gather_row_lse", k_row_lse<uint16_t>, dim3(n_rows), dim3(GT), st, (const uint16_t*)logits,
                         vocab, lse);
    else
      KDA_LAUNCH("gather_row_lse", k_row_lse<float>, dim3(n_rows), dim3(GT), st, (const float*)logits, vocab,
                         lse);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (n_pos > 0) {
    const int nb = (int)((n_pos + 255) / 256);
    if (bf16)
      KDA_LAUNCH("gather_pos_logp", k_pos_logp<uint16_t>, dim3(nb), dim3(256), st, (const uint16_t*)logits,
                         vocab, pos_row, pos_tgt, n_pos, lse, logp);
    else
      KDA_LAUNCH("gather_pos_logp", k_pos_logp<float>, dim3(nb), dim3(256), st, (const float*)logits, vocab,
                         pos_row, pos_tgt, n_pos, lse, logp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gather_bwd(const void* logits, bool bf16, int64_t n_rows, int vocab,
                             const float* lse, const int* row_pos_ptr, const int* row_pos_idx,
                             const int* pos_tgt, const float* dlogp, void* dlogits,
                             hipStream_t st) {
  if (n_rows <= 0) return hipSuccess;
  if (bf16)
    KDA_LAUNCH("gather_row_grad", k_row_grad<uint16_t>, dim3(n_rows), dim3(GT), st, (const uint16_t*)logits,
                       vocab, lse, row_pos_ptr, row_pos_idx, pos_tgt, dlogp, (uint16_t*)dlogits);
  else
    KDA_LAUNCH("gather_row_grad", k_row_grad<float>, dim3(n_rows), dim3(GT), st, (const float*)logits, vocab,
                       lse, row_pos_ptr, row_pos_idx, pos_tgt, dlogp, (float*)dlogits);
  return hipGetLastError();
}

}  // namespace kda
