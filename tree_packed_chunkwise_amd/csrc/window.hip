// window.hip -- state handoff between the calls of a sharing window (gfx950).
//
// Within a sharing window (thelatestinai.com Figure 3; HARTS abstract) a
// producer call computes the shared prefix once; consumer microbatches start
// from the producer's end states, and the gradients of those start states
// accumulate, microbatch by microbatch, into the producer's end-state
// gradients before the one producer backward.  These two kernels move and sum
// the D x D states between the calls; the calls themselves are kda_tree_fwd /
// kda_tree_bwd.  Every state is a block of `elems` floats moved as 16-byte
// vectors; sums run in a fixed order (deterministic).
#include <hip/hip_runtime.h>
#include <cstdint>
#include "timing.h"

namespace kda {

// dst[dst_idx[i]] = src[src_idx[i]] (a null index array is the identity)
__global__ __launch_bounds__(256) void k_state_copy(const float4* src, const int* sidx, float4* dst,
                                                    const int* didx, int64_t e4) {
  const int i = blockIdx.y;
  const int64_t s = sidx ? sidx[i] : i, d = didx ? didx[i] : i;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < e4; e += (int64_t)gridDim.x * 256)
    dst[d * e4 + e] = src[s * e4 + e];
}

// dst[d] = (accumulate ? dst[d] : 0) + sum over j in [ptr[d], ptr[d+1]) of src[idx[j]], j ascending
__global__ __launch_bounds__(256) void k_state_sum(const float4* src, const int* ptr, const int* idx,
                                                   float4* dst, int64_t e4, int accumulate) {
  const int d = blockIdx.y;
  const int j0 = ptr[d], j1 = ptr[d + 1];
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < e4; e += (int64_t)gridDim.x * 256) {
    float4 a = accumulate ? dst[d * e4 + e] : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = j0; j < j1; ++j) {
      const float4 x = src[(int64_t)idx[j] * e4 + e];
      a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
    }
    dst[d * e4 + e] = a;
  }
}

static int grid_x(int64_t e4) {
  const int64_t b = (e4 + 255) / 256;
  return (int)(b < 1024 ? (b < 1 ? 1 : b) : 1024);
}

hipError_t launch_state_copy(const float* src, const int* sidx, float* dst, const int* didx, int n,
                             int64_t elems, hipStream_t st) {
  if (n <= 0 || elems <= 0) return hipSuccess;
  const int64_t e4 = elems / 4;
  KDA_LAUNCH("kda_state_copy", k_state_copy, dim3(grid_x(e4), n), dim3(256), st, (const float4*)src,
             sidx, (float4*)dst, didx, e4);
  return hipGetLastError();
}

hipError_t launch_state_sum(const float* src, const int* ptr, const int* idx, int n_dst,
                            int64_t elems, int accumulate, float* dst, hipStream_t st) {
  if (n_dst <= 0 || elems <= 0) return hipSuccess;
  const int64_t e4 = elems / 4;
  KDA_LAUNCH("kda_state_sum", k_state_sum, dim3(grid_x(e4), n_dst), dim3(256), st,
             (const float4*)src, ptr, idx, (float4*)dst, e4, accumulate);
  return hipGetLastError();
}

}  // namespace kda
