// gemm.h -- block-cooperative small GEMMs on gfx950 matrix cores.
//
// C[M][N] = sum_k A(i,k) B(k,j) for operands reached through accessor
// functors (usually LDS reads, possibly with a decay factor applied), with
// fp32 accumulation on v_mfma_f32_16x16x32_bf16.  Each fp32 operand value x is
// split into hi = bf16(x) and lo = bf16(x - hi) and the product is formed as
// hi*hi + hi*lo + lo*hi, which keeps about 16 mantissa bits per product (a
// single bf16 rounding per operand would cost ~1.6e-3 relative error, most of
// the 2e-3 budget of the whole path).
//
// The M x N output is cut into 16 x 16 tiles dealt round-robin to the waves of
// the block; out(i, j, value) is called exactly once per output element, by
// the lane that owns it.  M and N must be multiples of 16; K is arbitrary
// (accessors are never called with k >= K).  A k-step of 32 whose range
// [kb, kb+32) is empty for a tile (as reported by `kskip`) is skipped.
#pragma once

#include <hip/hip_runtime.h>

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct NoSkip {
  __device__ bool operator()(int, int, int) const { return false; }
};

__device__ inline void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = (__bf16)x;
  lo = (__bf16)(x - (float)hi);
}

template <int M, int N, int K, int NWAVES, class FA, class FB, class FO, class FS = NoSkip>
__device__ inline void gemm3(const FA& A, const FB& B, const FO& out, const FS& kskip = FS()) {
  static_assert(M % 16 == 0 && N % 16 == 0, "tile");
  constexpr int TN = N / 16;
  constexpr int NT = (M / 16) * TN;
  constexpr int KS = (K + 31) / 32;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int kq = (lane >> 4) * 8;
  for (int t = wave; t < NT; t += NWAVES) {
    const int i0 = (t / TN) * 16;
    const int j0 = (t % TN) * 16;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int ks = 0; ks < KS; ++ks) {
      const int kb = ks * 32;
      if (kskip(i0, j0, kb)) continue;
      bf16x8 ah, al, bh, bl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kk = kb + kq + e;
        float a = 0.f, b = 0.f;
        if (K % 32 == 0 || kk < K) {
          a = A(i0 + l16, kk);
          b = B(kk, j0 + l16);
        }
        __bf16 h, l;
        split_bf16(a, h, l);
        ah[e] = h;
        al[e] = l;
        split_bf16(b, h, l);
        bh[e] = h;
        bl[e] = l;
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) out(i0 + (lane >> 4) * 4 + r, j0 + l16, acc[r]);
  }
}

}  // namespace kda
