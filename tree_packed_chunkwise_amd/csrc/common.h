// common.h -- shared device-side declarations of the KDA tree kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Device views of the uploaded plan tables (int32).
struct DevPlan {
  const int* round_seq_ptr;
  const int* seq_chunk_ptr;
  const int* seq_row_ptr;
  const int* seq_init_kind;
  const int* seq_init_idx;
  const int* seq_leaf;
  const int* seq_lpt;      // launch order of a round's sequences (most chunks first)
  const int* chunk_seq;
  const int* chunk_row0;
  const int* chunk_len;
  const int* chunk_save;
  const int* chunk_nrep;
  const int* chunk_rep0;
  const int* chunk_round;
  const int* row_index;
  const int* out_row;
  const int* buf_cons_ptr;
  const int* buf_cons;
  const int* buf_chunk;
  const int* rep_row;
  const int* rep_ptr;
  const int* rep_slot;
  const int* root_seq_ptr;
  const int* root_seq;
};

// Chunk images.  The state-independent part of every chunk step is computed
// once, fully parallel, by the chunk pass (kda_prep.hip) and stored per
// (chunk, head) as the exact LDS image that a round kernel's state phase
// reads: the round kernels copy it verbatim (16-byte vectors) and never touch
// q, k, g or the exponentials on their sequential path.  fp16 arrays are
// unpadded, their rows swizzled in 8-byte pieces (chunk.h swz) so that
// matrix-core fragment reads do not collide in LDS banks; every array is a
// multiple of 16 bytes.
//
// Forward image (BC rows, head dim D):
//   Qt  [BC][D]     q e^Gam                 Kn  [BC][D]    -k e^Gam
//   KhT [D][BC]     (k e^(Gam_C - Gam))^T   L   [BC][BC]   -A (strict lower; every reader
//                                                           subtracts A times something)
//   P   [BC][BC]    P (lower)               Td  [BC][24]   (I + diag(beta) A_II)^-1 per 16-row block
//   gc  [D] fp32    e^Gam_C                 beta [BC] fp32     orow [BC] int (-1: no output)
//   V   [BC][D]     v in the input dtype, in 16x16 accumulator-order tiles
//                   (the region is sized for fp32)
// The reverse pass reads the same image (its transposed operands through
// transposing LDS reads).  Rows past the chunk hold zeros (Gam, and so e^Gam,
// stays flat there).
constexpr __host__ __device__ size_t fwd_image_head_bytes(int BC, int D) {
  return (size_t)2 * (2 * (size_t)BC * D + (size_t)D * BC + 2 * (size_t)BC * BC +
                      (size_t)BC * 24) +
         4 * (size_t)D + 8 * (size_t)BC;
}
// bytes of one forward image as stored (V sized for fp32) and as used for an
// input element size of `elem` bytes
constexpr __host__ __device__ size_t fwd_image_bytes(int BC, int D) {
  return fwd_image_head_bytes(BC, D) + 4 * (size_t)BC * D;
}
constexpr __host__ __device__ size_t fwd_image_used(int BC, int D, int elem) {
  return fwd_image_head_bytes(BC, D) + (size_t)elem * BC * D;
}

struct FwdArgs {
  DevPlan plan;
  int H;
  float scale;
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const float* h0;     // may be null
  float* o;
  float* h_leaf;
  _Float16* chunk_h;   // [n_chunks,H,D,D] start state of every chunk (fp16 copy)
  float* bufs;         // [n_buf,H,D,D]
  unsigned char* fimg; // [n_chunks,H] chunk images, stride fwd_image_bytes
};

struct BwdArgs {
  DevPlan plan;
  int H;
  float scale;
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const _Float16* chunk_h; // saved start state per chunk [n_chunks,H,D,D] (fp16 copy)
  const unsigned char* fimg;  // chunk images (the round reads the head, the gradient pass A, Td, V)
  const void* dO;
  const float* dh_leaf;   // may be null
  float* dq;
  float* dk;
  float* dv;
  float* dg;
  float* dbeta;
  float* dh0;
  float* dh_boundary;     // may be null
  void* dOp;              // [n_chunks,H] x (BC x D dO in 16x16 tiles, state_tile order),
                          // zero on replay rows and past the chunk
  _Float16* dy;           // [n_chunks,H] x (BC x D fp16 in 16x16 tiles, state_tile order)
  _Float16* dhc;          // [n_chunks,H,D,D] gradient of each chunk's end state (fp16 copy)
  float* slot;            // [n_seq,H,D,D] gradient of each sequence's start state
  float* rep_dq;          // [n_replay,H,D] gradients of replayed rows
  float* rep_dk;
  float* rep_dg;
  float* rep_dv;
  float* rep_db;          // [n_replay,H]
  int n_rounds;
  unsigned* gmax;         // [scale_words(n_rounds)] gradient-scale words (fp32 bits), see below
};

// The reverse pass runs each round in units scaled by a power of two s_r,
// chosen so that the largest upstream gradient the round takes in lies in
// [8, 16): the fp16 operands of the state-gradient products then keep their
// precision whatever the loss's scale (a loss averaged over many positions
// has gradients far below fp16's normal range, a scaled one far above it).
// The gradients a round takes in: its chunks' dO (times scale), the leaf
// states' gradients, and the start-state gradients of the sequences of later
// rounds that started from its handoff states.  Those and every gradient
// leave a round unscaled (fp32), so each round may have its own s_r.
// Maxima are kept as fp32 bits (non-negative floats order like their bits,
// so an integer atomic max gives the maximum in any order), each spread over
// SPREAD words (a writer picks one by its block index, so that atomics to
// one address do not queue up; a reader takes the maximum of all of them).
// Words of gmax, R = n_rounds:
//   [0, S)                       max |dh_leaf|
//   [S + r S, S + (r + 1) S)     max |dO| over the chunks of round r  (the dO gather)
//   [S + R S + r S, ...)         max |start-state gradient| written by round r
//   [S + 2 R S + r]              max over the start-state words of rounds r' > r (round r)
//   [S + 2 R S + R + r]          s_r                                  (round r)
constexpr int SPREAD = 64;
constexpr __host__ __device__ size_t scale_words(int R) { return (size_t)SPREAD * (1 + 2 * R) + 2 * R; }
__device__ inline unsigned* leaf_words(unsigned* g) { return g; }
__device__ inline unsigned* dO_words(unsigned* g, int r) { return g + SPREAD * (1 + r); }
__device__ inline unsigned* slot_words(unsigned* g, int R, int r) { return g + SPREAD * (1 + R + r); }
__device__ inline unsigned* suffix_word(unsigned* g, int R, int r) { return g + SPREAD * (1 + 2 * R) + r; }
__device__ inline unsigned* scale_word(unsigned* g, int R, int r) { return g + SPREAD * (1 + 2 * R) + R + r; }
// maximum of SPREAD words, by one whole wave (every lane returns it)
__device__ inline float spread_max(const unsigned* w) {
  float m = __uint_as_float(w[threadIdx.x & 63]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  return m;
}
inline __device__ float pow2_scale(float m) {
  if (!(m > 0.f) || !(m < INFINITY)) return 1.f;
  int e = 0;
  (void)frexpf(m, &e);    // m = f 2^e, f in [0.5, 1)
  int k = 4 - e;
  k = k < -120 ? -120 : (k > 120 ? 120 : k);
  return ldexpf(1.f, k);
}
// the scale of round r, by whole waves of the round's own kernel; `later`
// receives the maximum over the later rounds' start-state gradients
inline __device__ float round_scale(unsigned* gm, int R, int r, float attn_scale, float* later) {
  float suf = 0.f;
  if (r + 1 < R) suf = fmaxf(__uint_as_float(*suffix_word(gm, R, r + 1)), spread_max(slot_words(gm, R, r + 1)));
  *later = suf;
  return pow2_scale(fmaxf(fmaxf(spread_max(dO_words(gm, r)) * attn_scale, spread_max(leaf_words(gm))), suf));
}

// Tree-ancestor attention (attn.hip): plan tables (see plan.h) and tensors.
struct AttnArgs {
  const int* seg_row;
  const int* seg_len;
  const int* anc_ptr;
  const int* anc;
  const int* tile_seg;
  const int* tile_off;
  const int* qorder;
  const int* kq_ptr;
  const int* kq;
  const int* kw_tile;
  const int* kw_q0;
  const int* kw_nq;
  const int* kw_slot;
  const int* ks_tile;
  const int* ks_slot0;
  const int* ks_n;
  int H;
  float scale;
  const uint16_t* q;  // bf16 [N][H][D]
  const uint16_t* k;
  const uint16_t* v;
  float* o;           // [N][H][D]
  float* lse;         // [N][H]
  const uint16_t* dO; // bf16 [N][H][D]
  const float* oc;    // forward output (backward input)
  const float* lsec;
  float* delta;       // [N][H]
  float* dq;
  float* dk;
  float* dv;
  float* part;        // [n_slots][H][2][64][D] partial dk, dv
};

// A plan value at a block-uniform index, read through the constant address
// space so that it becomes a scalar load: the plan tables are never written
// while a kernel runs.  A vector load of it would share the vector-memory
// wait counter with the block's image prefetch and result stores, and the
// wait for its value would wait for all of them.
template <typename T>
__device__ inline T ld_uni(const T* p, size_t i) {
  return ((const __attribute__((address_space(4))) T*)p)[i];
}

// One input element as fp32, loaded through the global address space (every
// input lives in device memory; the compiler cannot always infer that, and a
// flat load counts against both wait counters).
template <typename T>
using gptr = const __attribute__((address_space(1))) T*;
inline __device__ float ld_in(const float* p, size_t i) { return ((gptr<float>)p)[i]; }
inline __device__ float ld_in(const uint16_t* p, size_t i) {
  return __uint_as_float(((uint32_t)((gptr<uint16_t>)p)[i]) << 16);
}

}  // namespace kda
